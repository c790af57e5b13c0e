"""The C-ABI library without a GPU: it loads, exports every function the header
declares, reports its ABI revision, plans splits by its documented rules and
rejects bad arguments before anything reaches a device.  No compute calls."""

import ctypes
import os
import re

import numpy as np
import pytest

import fp8_kv_paged_attn_amd as pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn_e4m3.h")

PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EALIGN, PA_EDEVICE, PA_EHIP, PA_EPLAN = (
    0, -1, -2, -3, -4, -5, -6, -7)
PA_ESCRATCH = -8


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(pa.LIB_PATH):
        from fp8_kv_paged_attn_amd import build

        build.build()
    return pa.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == set(pa.EXPORTS), names
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_abi_and_status(L):
    assert L.paged_attn_abi_version() == pa.ABI_VERSION == 3
    for rc in (PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EALIGN, PA_EDEVICE, PA_EHIP,
               PA_EPLAN, PA_ESCRATCH, 12345):
        s = L.paged_attn_status_string(rc)
        assert s and len(s) > 1


def mfma_slots_fit(p) -> bool:
    """The MFMA kernel's rule: a split of T positions in pages of P tokens
    needs (T - 1) // P + 2 page slots (token ids: T), within 1,024 slots at
    head_dim 256 and 2,048 at 128."""
    T = p.tokens_per_split
    need = T if p.selection == pa.PA_SELECTION["tokens"] else (T - 1) // p.page_size + 2
    return need <= (1024 if p.head_dim == 256 else 2048)


@pytest.mark.parametrize("max_tokens,rows,units,D,page,sel,cus,req", [
    (2048, 12, 1, 256, 800, "dense", 256, 4), (8192, 48, 1, 256, 3296, "dense", 0, 0),
    (65536, 48, 1, 256, 3296, "dense", 0, 0), (131072, 48, 1, 256, 3296, "dense", 0, 0),
    (262144, 48, 1, 256, 3456, "dense", 0, 0), (2048, 48, 32, 128, 64, "blocks", 0, 0),
    (1, 6, 1, 256, 16, "dense", 0, 0), (0, 6, 1, 256, 16, "dense", 0, 0),
    (300, 4, 2, 128, 7, "dense", 0, 7), (64, 48, 1, 256, 1, "dense", 0, 9),
    (100000, 48, 3, 256, 1616, "dense", 80, 0), (262144, 48, 1, 256, 3456, "dense", 0, 100000),
    (32960, 96, 8, 256, 1600, "dense", 0, 0), (32960, 49, 8, 256, 1600, "dense", 0, 0),
    (2048, 48, 32, 128, 64, "tokens", 0, 0), (4096, 48, 256, 256, 64, "tokens", 0, 0),
    (262144, 48, 1, 256, 1, "dense", 0, 0), (262144, 48, 1, 256, 1, "dense", 0, 1),
    (20000, 48, 1, 128, 1, "blocks", 0, 1), (70000, 12, 1, 256, 2, "dense", 0, 0),
    (16384, 48, 1, 256, 3296, "dense", 0, 0), (32768, 48, 1, 256, 3296, "dense", 0, 0),
    (8192, 40, 1, 256, 3296, "dense", 0, 0), (8192, 20, 2, 256, 64, "dense", 0, 0),
    (4096, 48, 2, 128, 64, "blocks", 0, 0), (512, 48, 4, 256, 16, "tokens", 0, 0),
])
def test_plan_rules(L, max_tokens, rows, units, D, page, sel, cus, req):
    p = pa.plan(max_tokens, rows, units, D, page, sel, num_cus=cus, splits=req)
    S, T = p.num_splits, p.tokens_per_split
    tiles = max(1, -(-max_tokens // 64))
    assert T % 64 == 0 and T >= 64 and 1 <= S <= 65535
    assert S * T >= max_tokens
    if max_tokens > 0:
        assert (S - 1) * T < max_tokens, "no split may lie wholly past max_tokens"
    assert mfma_slots_fit(p), "every plan runs on the MFMA kernel"
    ch = p.rows_per_workgroup
    assert ch in (16, 32, 48)
    if ch != 48:
        # finer row chunks only for short lists (fewer than two 128-token
        # steps per 48-row workgroup), at most one workgroup per compute unit,
        # splits of at most 3 steps (16 rows) or 4 (32 rows), a split count
        # that keeps the (split, unit) pairs a multiple of 8 (or below 8), and
        # only where they cut a unit into more chunks
        c = cus if cus > 0 else 256
        assert not req and rows > ch
        assert S * units * -(-rows // ch) <= c and T <= (384 if ch == 16 else 512)
        assert (S * units) % 8 == 0 or S * units < 8
        p48 = -(-tiles // min(max(1, c // (units * -(-rows // 48))),
                              max(1, -(-max_tokens // 128)))) * 64
        assert p48 < 256
        assert (p.ws_acc_bytes, p.ws_stat_bytes) == (S * rows * units * D * 4, S * rows * units * 4)
        return
    # the slot cap only ever raises the count: the uncapped rule's count is a lower bound
    if req:
        want = min(req, tiles)
    else:
        c = cus if cus > 0 else 256
        want = min(max(1, c // (units * -(-rows // 48))), max(1, -(-max_tokens // 128)))
    T0 = -(-tiles // want) * 64
    S0 = max(1, -(-max_tokens // T0))
    assert S >= S0
    if S > S0:
        # raised only because the uncapped split overflowed the slot cache, and
        # then to the fewest splits of the longest split that fits
        slots = 1024 if D == 256 else 2048
        cap = slots if sel == "tokens" else (slots - 1) * page
        assert T0 > cap and T == cap // 64 * 64
    else:
        assert T == T0
    assert (p.max_tokens, p.rows_per_kv_unit, p.num_kv_units, p.head_dim, p.page_size,
            p.selection) == (max_tokens, rows, units, D, page, pa.PA_SELECTION[sel])
    assert p.ws_acc_bytes == S * rows * units * D * 4
    assert p.ws_stat_bytes == S * rows * units * 4
    assert p.kernel == 0


@pytest.mark.parametrize("units", [1, 2, 3, 5, 6, 7, 8, 32, 255, 256])
def test_plan_fills_at_most_one_round(L, units):
    """Planner-chosen counts never put more workgroups than compute units
    (while one split per unit fits): a few left over would run as a second
    round and double the call."""
    for ctx in (8192, 65536, 131072, 262144):
        p = pa.plan(ctx, 48, units, 256, 3296, num_cus=256)
        chunks = -(-48 // p.rows_per_workgroup)
        assert p.num_splits * units * chunks <= 256, (ctx, units, p)


def test_plan_counts_row_chunks(L):
    # 8 units of 96 rows = 16 workgroups per split: 16 splits fill 256 CUs
    assert pa.plan(32960, 96, 8, 256, 1600, num_cus=256).num_splits == 16
    # 8 units of 48 rows: 32 splits wanted; 1,088 tokens each cover 32,960 in 31
    assert pa.plan(32960, 48, 8, 256, 1600, num_cus=256).num_splits == 31


@pytest.mark.parametrize("max_tokens,rows,units,req,expect", [
    (8192, 48, 1, 0, (64, 128, 16)),      # 3 chunks x 64 splits = 192 workgroups
    (16384, 48, 1, 0, (64, 256, 16)),     # 16-row chunks with two steps per split
    (24576, 48, 1, 0, (64, 384, 16)),     # 77 splits of 320 would split pairs over XCDs
    (32768, 48, 1, 0, (128, 256, 32)),    # 16 rows would need 448-token splits
    (49152, 48, 1, 0, (128, 384, 32)),    # 48 rows: 192-token splits, under two steps
    (53248, 48, 1, 0, (208, 256, 48)),    # two steps per 48-row workgroup
    (65536, 48, 1, 0, (256, 256, 48)),    # two steps per 48-row workgroup already
    (8192, 48, 1, 64, (64, 128, 48)),     # a requested count keeps 48-row chunks
    (8192, 12, 1, 0, (64, 128, 48)),      # one chunk of 16 rows either way
    (8192, 20, 1, 0, (64, 128, 16)),      # 16 + 4 rows
    (8192, 48, 2, 0, (32, 256, 16)),      # 2 units x 3 chunks x 32 splits of 256 tokens
])
def test_plan_row_chunks_for_short_lists(L, max_tokens, rows, units, req, expect):
    p = pa.plan(max_tokens, rows, units, 256, 3296, num_cus=256, splits=req)
    assert (p.num_splits, p.tokens_per_split, p.rows_per_workgroup) == expect
    assert pa.plan(max_tokens, rows, units, 256, 3296, "batch", num_cus=256).rows_per_workgroup == 48


def test_plan_raises_splits_to_fit_the_slot_cache(L):
    # one page per token: a 1,024-token split would need 1,025 slots; 960 fit
    p = pa.plan(262144, 48, 1, 256, 1, num_cus=256)
    assert (p.tokens_per_split, p.num_splits) == (960, 274)
    # 4,096 token ids over 256 units want one split each, but 1,024 ids fit a split
    p = pa.plan(4096, 48, 256, 256, 64, "tokens", num_cus=256)
    assert (p.tokens_per_split, p.num_splits) == (1024, 4)
    # head_dim 128 keeps twice the slots
    p = pa.plan(4096, 48, 256, 128, 64, "tokens", num_cus=256)
    assert (p.tokens_per_split, p.num_splits) == (2048, 2)


def test_plan_rejects(L):
    out = pa.PaPlan()
    f = L.paged_attn_plan
    assert f(-1, 48, 1, 256, 16, 0, 0, 0, ctypes.byref(out)) == PA_EINVAL
    assert f(10, 0, 1, 256, 16, 0, 0, 0, ctypes.byref(out)) == PA_EINVAL
    assert f(10, 4, 0, 256, 16, 0, 0, 0, ctypes.byref(out)) == PA_EINVAL
    assert f(10, 4, 1, 256, 16, 0, 0, -2, ctypes.byref(out)) == PA_EINVAL
    assert f(10, 4, 1, 256, 0, 0, 0, 0, ctypes.byref(out)) == PA_EINVAL      # page size
    assert f(10, 4, 1, 256, 16, 4, 0, 0, ctypes.byref(out)) == PA_EINVAL     # selection
    assert f(10, 4, 1, 256, 16, 0, 0, 0, None) == PA_EINVAL
    # a count past 65,535 splits: two billion tokens in one-token pages
    assert f(2 ** 31 - 1, 4, 1, 256, 1, 0, 0, 0, ctypes.byref(out)) == PA_EUNSUPPORTED


@pytest.mark.parametrize("cap,rows,units,D,page,cus,req", [
    (32 * 1024, 96, 8, 256, 3296, 256, 0), (32 * 1024, 48, 8, 256, 3296, 256, 0),
    (512, 96, 4, 256, 64, 0, 0), (4096, 96, 300, 256, 64, 256, 0), (1 << 20, 12, 2, 256, 1, 256, 0),
    (700, 6, 1, 128, 16, 256, 5), (0, 6, 3, 256, 16, 256, 0),
])
def test_plan_batch_rules(L, cap, rows, units, D, page, cus, req):
    """A batch plan: num_splits counts the splits of all units (one workgroup per
    compute unit and 48-row chunk, or as requested), at least enough for every
    unit at full length at the longest span the MFMA kernel takes."""
    p = pa.plan(cap, rows, units, D, page, "batch", num_cus=cus, splits=req)
    S, T = p.num_splits, p.tokens_per_split
    slots = 1024 if D == 256 else 2048
    assert T % 64 == 0 and T >= 64
    assert T == min((slots - 1) * page // 64 * 64, max(1, -(-cap // 64)) * 64)
    assert mfma_slots_fit(p)
    chunks = -(-rows // 48)
    want = req if req else -(-(cus or 256) // chunks)
    assert S == max(want, units * -(-cap // T), 1)
    assert p.ws_acc_bytes == S * rows * D * 4 and p.ws_stat_bytes == S * rows * 4
    assert p.ws_index_bytes == (units + 1) * 4


def test_ragged_plan_rule_covers_every_length():
    """The device's ragged rule (re-derived on the host) always fits the splits:
    sum_u ceil(L_u / T) <= S for any lengths up to the capacity, with T on the
    tile and at most the plan's span."""
    from tests import gpu_util as gu

    rng = np.random.default_rng(0x5A7)
    for _ in range(400):
        B = int(rng.integers(1, 40))
        Hkv = int(rng.integers(1, 4))
        q = int(rng.integers(1, 17))
        cap = int(rng.integers(1, 200000))
        tcap = int(rng.choice([64, 960, 1024, 4096, 65472]))
        S = B * Hkv * -(-cap // tcap) + int(rng.integers(0, 300))
        lens = rng.integers(-5, cap + 50, size=(B, q))
        lens[rng.random((B, q)) < 0.2] = 0
        T, index = gu.ragged_plan(lens, cap, Hkv, S, tcap)
        assert T % 64 == 0 and 64 <= T <= max(tcap, 64)
        assert index[-1] <= S and np.all(np.diff(index) >= 0)
        L = np.repeat(np.clip(lens, 0, cap).max(axis=1), Hkv)
        assert np.all(np.diff(index) * T >= L), "a unit's splits cover its length"


def test_build_id_matches_sources(L):
    from fp8_kv_paged_attn_amd import build

    assert pa.build_id() == build.source_hash()
    assert len(pa.build_id()) == 16


def test_binding_refuses_a_library_built_from_other_sources(L, monkeypatch):
    from fp8_kv_paged_attn_amd import build

    monkeypatch.setattr(pa, "_LIB", None)
    monkeypatch.setattr(build, "source_hash", lambda: "0" * 16)
    with pytest.raises(RuntimeError, match="other sources"):
        pa.lib()


def test_scales_are_host_values():
    """Scales are folded on the host: a tensor on a device is refused before any
    call, so nothing reads it back (no synchronisation, capturable calls)."""
    import torch

    assert pa._scale(torch.tensor(0.5), "k_scale") == 0.5
    assert pa._scale(np.float32(2.25), "v_scale") == 2.25
    with pytest.raises(ValueError, match="host scalar"):
        pa._scale(torch.tensor(0.5, device="meta"), "k_scale")
    with pytest.raises(ValueError, match="one element"):
        pa._scale(torch.ones(2), "k_scale")
    with pytest.raises(ValueError, match="finite"):
        pa._scale(float("nan"), "k_scale")


# Fake, 16-byte-aligned addresses: every call below is rejected by a host check
# before any HIP call, so they are never dereferenced.  The tests still stay
# off machines with a GPU, where a wrongly accepted call could reach it.
A = 0x10000
no_device = pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="fake pointers; CPU only")


class Call:
    """A valid-looking dense verify call whose fields the tests spoil one at a time."""

    def __init__(self):
        self.q = A
        self.pool = pa.PaKvPool(A * 2, A * 3, 3296 * 256, 256, 256, 64, 3296)
        self.table, self.entries = A * 4, 3
        self.lens, self.max_tokens = A * 5, 8192
        self.q_rows, self.H, self.Hkv, self.D = 8, 6, 1, 256
        self.sm, self.ks = 0.0625, 0.37
        self.plan = pa.plan(8192, 48, 1, 256, 3296)
        S = self.plan.num_splits
        self.ws = pa.PaWorkspace(A * 6, A * 7, A * 8, S * 48 * 256 * 4, S * 48 * 4)

    def __call__(self, L):
        return L.paged_attn_verify_e4m3(self.q, ctypes.byref(self.pool), self.table, self.entries,
                                        self.lens, self.max_tokens, self.q_rows, self.H, self.Hkv,
                                        self.D, self.sm, self.ks, ctypes.byref(self.plan),
                                        ctypes.byref(self.ws), None)


def _spoil(L, attr, value, expect, sub=None):
    c = Call()
    tgt = getattr(c, sub) if sub else c
    setattr(tgt, attr, value)
    assert c(L) == expect, (attr, value)


@no_device
def test_verify_rejects_bad_arguments(L):
    _spoil(L, "q", None, PA_EINVAL)
    _spoil(L, "table", None, PA_EINVAL)
    _spoil(L, "lens", None, PA_EINVAL)
    _spoil(L, "k_pool", None, PA_EINVAL, sub="pool")
    _spoil(L, "D", 64, PA_EUNSUPPORTED)
    _spoil(L, "q_rows", 9, PA_EUNSUPPORTED)
    _spoil(L, "q_rows", 0, PA_EINVAL)
    _spoil(L, "Hkv", 4, PA_EINVAL)                 # 6 % 4 != 0
    _spoil(L, "H", 12, PA_EUNSUPPORTED)            # 8 x 12 rows per KV head > 48
    c = Call()                                     # more than 65,536 heads
    c.H, c.Hkv = 6 * 16384, 16384
    assert c(L) == PA_EUNSUPPORTED
    _spoil(L, "q", A + 8, PA_EALIGN)
    _spoil(L, "k_pool", A * 2 + 4, PA_EALIGN, sub="pool")
    _spoil(L, "token_stride", 264 - 4, PA_EALIGN, sub="pool")
    _spoil(L, "page_size", 0, PA_EINVAL, sub="pool")
    _spoil(L, "entries", 2, PA_EINVAL)             # 2 x 3296 < 8192
    _spoil(L, "max_tokens", -1, PA_EINVAL)
    _spoil(L, "ks", 0.0, PA_EINVAL)
    _spoil(L, "ks", float("nan"), PA_EINVAL)
    _spoil(L, "sm", float("inf"), PA_EINVAL)
    _spoil(L, "sm", -0.0625, PA_EINVAL)
    _spoil(L, "sm", 0.0, PA_EINVAL)
    _spoil(L, "sm", 1e-40, PA_EINVAL)            # folded scale underflows
    _spoil(L, "max_tokens", 8000, PA_EPLAN)        # plan made for 8192
    _spoil(L, "tokens_per_split", 100, PA_EPLAN, sub="plan")
    _spoil(L, "num_splits", 1, PA_EPLAN, sub="plan")
    _spoil(L, "kernel", 7, PA_EPLAN, sub="plan")
    _spoil(L, "page_size", 3200, PA_EPLAN, sub="plan")             # made for other pages
    _spoil(L, "selection", 1, PA_EPLAN, sub="plan")                # made for blocks
    _spoil(L, "tokens_per_split", 1 << 30, PA_EPLAN, sub="plan")   # S*T past INT32_MAX
    _spoil(L, "num_splits", 200, PA_EPLAN, sub="plan")              # splits wholly past the end
    _spoil(L, "rows_per_workgroup", 24, PA_EPLAN, sub="plan")       # chunks of 16, 32 or 48 rows
    _spoil(L, "rows_per_workgroup", 64, PA_EPLAN, sub="plan")
    for ch in (0, 16, 32, 48):                                      # 0 reads as 48
        _spoil(L, "rows_per_workgroup", ch, PA_EDEVICE, sub="plan")
    _spoil(L, "acc_bytes", 1024, PA_EWORKSPACE, sub="ws")
    _spoil(L, "stat_bytes", 4, PA_EWORKSPACE, sub="ws")
    _spoil(L, "sum", None, PA_EINVAL, sub="ws")


@no_device
def test_qsa_and_combine_reject_bad_arguments(L):
    pool = pa.PaKvPool(A * 2, A * 3, 64 * 256, 256, 128, 8192, 64)
    p = pa.plan(32 * 64, 48, 32, 128, 64, "blocks")
    ws = pa.PaWorkspace(A * 6, A * 7, A * 8, p.ws_acc_bytes, p.ws_stat_bytes)

    def qsa(**kw):
        a = dict(q=A, table=A * 4, maxb=512, sel=A * 9, topk=32, lens=A * 5, B=16, qr=4, H=24,
                 Hkv=2, D=128, sm=0.088, ks=0.5)
        a.update(kw)
        return L.qsa_sparse_verify_e4m3(a["q"], ctypes.byref(pool), a["table"], a["maxb"],
                                        a["sel"], a["topk"], a["lens"], a["B"], a["qr"], a["H"],
                                        a["Hkv"], a["D"], a["sm"], a["ks"], ctypes.byref(p),
                                        ctypes.byref(ws), None)

    assert qsa(sel=None) == PA_EINVAL
    assert qsa(topk=0) == PA_EINVAL
    assert qsa(B=0) == PA_EINVAL
    assert qsa(topk=31) == PA_EPLAN
    assert qsa(B=8) == PA_EPLAN
    assert qsa(ks=-0.5) == PA_EINVAL
    assert qsa(H=96) == PA_EUNSUPPORTED
    assert L.paged_attn_combine_fp32(A, A, A, 0, 48, 256, 1.0, A, None) == PA_EINVAL
    assert L.paged_attn_combine_fp32(A, A, A, 4, 48, 256, float("nan"), A, None) == PA_EINVAL
    assert L.paged_attn_combine_fp32(None, A, A, 4, 48, 256, 1.0, A, None) == PA_EINVAL
    assert L.paged_attn_combine_fp32(A, A, A, 4, 48, 256, 1.0, None, None) == PA_EINVAL


@no_device
def test_qsa_tokens_rejects_bad_arguments(L):
    """The token-id entry: the plan is made for num_sel list positions (not
    num_sel * page_size), and a device-free valid call reaches PA_EDEVICE."""
    pool = pa.PaKvPool(A * 2, A * 3, 64 * 256, 256, 128, 8192, 64)
    p = pa.plan(2048, 48, 32, 128, 64, "tokens")
    ws = pa.PaWorkspace(A * 6, A * 7, A * 8, p.ws_acc_bytes, p.ws_stat_bytes)

    def tok(**kw):
        a = dict(q=A, table=A * 4, maxb=512, sel=A * 9, n=2048, lens=A * 5, B=16, qr=4, H=24,
                 Hkv=2, D=128, sm=0.088, ks=0.5, plan=p)
        a.update(kw)
        return L.qsa_sparse_verify_tokens_e4m3(a["q"], ctypes.byref(pool), a["table"],
                                               a["maxb"], a["sel"], a["n"], a["lens"], a["B"],
                                               a["qr"], a["H"], a["Hkv"], a["D"], a["sm"],
                                               a["ks"], ctypes.byref(a["plan"]),
                                               ctypes.byref(ws), None)

    assert tok() == PA_EDEVICE
    assert tok(sel=None) == PA_EINVAL
    assert tok(n=0) == PA_EINVAL
    assert tok(n=32) == PA_EPLAN                        # the block entry's list length
    assert tok(plan=pa.plan(4096, 48, 32, 128, 64, "tokens")) == PA_EPLAN
    assert tok(plan=pa.plan(2048, 48, 32, 128, 64, "blocks")) == PA_EPLAN
    # a hand-made split longer than the MFMA kernel's slot cache runs only on
    # the plain kernel, when asked for
    long = pa.plan(2048, 48, 32, 128, 64, "tokens", splits=1)
    long.num_splits, long.tokens_per_split = 1, 2112
    long.ws_acc_bytes, long.ws_stat_bytes = p.ws_acc_bytes, p.ws_stat_bytes
    assert tok(plan=long) == PA_EPLAN
    long.kernel = pa.PA_KERNEL["mfma"]
    assert tok(plan=long) == PA_EPLAN
    long.kernel = pa.PA_KERNEL["simple"]
    assert tok(plan=long) == PA_EDEVICE
    assert tok(B=8) == PA_EPLAN
    assert tok(q=A + 8) == PA_EALIGN
    assert tok(ks=float("inf")) == PA_EINVAL
    assert tok(H=96) == PA_EUNSUPPORTED


@no_device
def test_valid_call_without_device_reports_edevice(L):
    assert Call()(L) == PA_EDEVICE


@no_device
def test_noalloc_entry_checks_before_any_device_call(L):
    """The allocation-free entry checks its arguments like the workspace entry,
    refuses a plan whose partials exceed the fixed scratch (PA_ESCRATCH), and
    only then looks for a device."""
    c = Call()
    out = A * 9

    def call(plan=None, out=out, vs=1.9, max_tokens=8192):
        p = plan or c.plan
        return L.paged_attn_verify_noalloc_e4m3(c.q, ctypes.byref(c.pool), c.table, c.entries,
                                                c.lens, max_tokens, c.q_rows, c.H, c.Hkv, c.D,
                                                c.sm, c.ks, vs, ctypes.byref(p), out, None)

    assert call() == PA_EDEVICE
    assert call(out=None) == PA_EINVAL
    assert call(out=A * 9 + 4) == PA_EALIGN
    assert call(vs=float("inf")) == PA_EINVAL
    assert call(max_tokens=8000) == PA_EPLAN
    big = pa.plan(8192, 48, 1, 256, 3296, splits=128)
    assert big.num_splits * 48 * 258 * 4 <= pa.NOALLOC_SCRATCH_BYTES
    assert call(plan=big) == PA_EDEVICE
    pool = pa.PaKvPool(A * 2, A * 3, 4096 * 256, 256, 256, 64, 4096)
    huge = pa.plan(1 << 15, 48, 1, 256, 4096, splits=512)
    assert huge.num_splits * 48 * 258 * 4 > pa.NOALLOC_SCRATCH_BYTES
    assert L.paged_attn_verify_noalloc_e4m3(c.q, ctypes.byref(pool), c.table, 8, c.lens,
                                            1 << 15, 8, 6, 1, 256, c.sm, c.ks, 1.0,
                                            ctypes.byref(huge), out, None) == PA_ESCRATCH


def test_verify_batch_rejects_bad_arguments(L):
    pool = pa.PaKvPool(k_pool=0x10000, v_pool=0x20000, page_stride=256 * 64, token_stride=256,
                       head_stride=256, num_pages=64, page_size=64)
    p = pa.PaPlan()
    assert L.paged_attn_plan(64 * 8, 96, 4, 256, 64, 3, 0, 0, ctypes.byref(p)) == PA_OK
    ws = pa.PaWorkspace(acc=0x30000, max=0x40000, sum=0x50000, acc_bytes=1 << 40,
                        stat_bytes=1 << 40, index=0x70000, index_bytes=1 << 20)
    A = ctypes.c_void_p(0x60000)
    f = L.paged_attn_verify_batch_e4m3

    def call(q=A, table=A, mb=8, lens=A, B=4, qr=16, H=6, Hkv=1, D=256, sm=0.0625, ks=1.0,
             plan=p, w=ws):
        return f(q, ctypes.byref(pool), table, mb, lens, B, qr, H, Hkv, D, sm, ks,
                 ctypes.byref(plan), ctypes.byref(w), None)

    assert call(q=None) == PA_EINVAL
    assert call(table=None) == PA_EINVAL
    assert call(B=0) == PA_EINVAL
    assert call(mb=0) == PA_EINVAL
    assert call(qr=17) == PA_EUNSUPPORTED
    assert call(qr=16, H=12, Hkv=1) == PA_EUNSUPPORTED        # 192 rows per KV head
    assert call(H=7, Hkv=2) == PA_EINVAL
    assert call(D=192) == PA_EUNSUPPORTED
    assert call(q=ctypes.c_void_p(0x60008)) == PA_EALIGN
    assert call(sm=-1.0) == PA_EINVAL
    assert call(mb=9) == PA_EPLAN                              # plan made for 8 blocks
    assert call(B=3) == PA_EPLAN                               # plan made for 4 units
    small = pa.PaWorkspace(acc=0x30000, max=0x40000, sum=0x50000, acc_bytes=16, stat_bytes=16,
                           index=0x70000, index_bytes=1 << 20)
    assert call(w=small) == PA_EWORKSPACE
    noidx = pa.PaWorkspace(acc=0x30000, max=0x40000, sum=0x50000, acc_bytes=1 << 40,
                           stat_bytes=1 << 40)
    assert call(w=noidx) == PA_EINVAL                           # the split index is missing
    shortidx = pa.PaWorkspace(acc=0x30000, max=0x40000, sum=0x50000, acc_bytes=1 << 40,
                              stat_bytes=1 << 40, index=0x70000, index_bytes=16)
    assert call(w=shortidx) == PA_EWORKSPACE                    # 4 units need 5 entries
    dense = pa.PaPlan()
    assert L.paged_attn_plan(64 * 8, 96, 4, 256, 64, 0, 0, 0, ctypes.byref(dense)) == PA_OK
    assert call(plan=dense) == PA_EPLAN                         # not a batch plan
    few = pa.PaPlan()
    assert L.paged_attn_plan(64 * 8, 96, 4, 256, 64, 3, 0, 0, ctypes.byref(few)) == PA_OK
    few.num_splits = 3
    assert call(plan=few) == PA_EPLAN                           # fewer splits than units
    fine = pa.PaPlan()
    assert L.paged_attn_plan(64 * 8, 96, 4, 256, 64, 3, 0, 0, ctypes.byref(fine)) == PA_OK
    fine.rows_per_workgroup = 16
    assert call(plan=fine) == PA_EPLAN                          # a batch takes 48-row chunks


@no_device
def test_verify_batch_without_device_reports_edevice(L):
    pool = pa.PaKvPool(k_pool=0x10000, v_pool=0x20000, page_stride=256 * 64, token_stride=256,
                       head_stride=256, num_pages=64, page_size=64)
    p = pa.PaPlan()
    assert L.paged_attn_plan(64 * 8, 96, 4, 256, 64, 3, 0, 0, ctypes.byref(p)) == PA_OK
    ws = pa.PaWorkspace(acc=0x30000, max=0x40000, sum=0x50000, acc_bytes=1 << 40,
                        stat_bytes=1 << 40, index=0x70000, index_bytes=1 << 20)
    A = ctypes.c_void_p(0x60000)
    assert L.paged_attn_combine_batch_fp32(ctypes.byref(ws), ctypes.byref(p), 4, 16, 6, 1, 256,
                                           1.0, A, None) == PA_EDEVICE
    assert L.paged_attn_verify_batch_e4m3(A, ctypes.byref(pool), A, 8, A, 4, 16, 6, 1, 256,
                                          0.0625, 1.0, ctypes.byref(p), ctypes.byref(ws),
                                          None) == PA_EDEVICE
    lse = L.paged_attn_combine_batch_fp32_lse
    args = (ctypes.byref(ws), ctypes.byref(p), 4, 16, 6, 1, 256, 1.0)
    assert lse(*args, A, None, None, None) == PA_EDEVICE
    assert lse(*args, None, ctypes.c_void_p(0x80000), ctypes.c_void_p(0x90000), None) == PA_EDEVICE
    assert lse(*args, None, None, None, None) == PA_EINVAL             # no output
    assert lse(*args, None, ctypes.c_void_p(0x80008), None, None) == PA_EALIGN   # out_fp32
    assert lse(*args, None, None, ctypes.c_void_p(0x90002), None) == PA_EALIGN   # lse
    assert lse(*args[:2], 4, 16, 6, 1, 64, 1.0, A, None, None, None) == PA_EUNSUPPORTED


def test_cache_write_rejects_bad_arguments(L):
    pool = pa.PaKvPool(k_pool=0x10000, v_pool=0x20000, page_stride=256 * 16, token_stride=256,
                       head_stride=256, num_pages=8, page_size=16)
    A = ctypes.c_void_p(0x60000)
    f = L.paged_attn_cache_write_e4m3

    def call(k=A, v=A, T=4, Hkv=1, D=256, slots=A, ks=0.5, vs=2.0, kv=pool):
        return f(k, v, T, Hkv, D, slots, ctypes.byref(kv), ks, vs, None)

    assert call(k=None) == PA_EINVAL
    assert call(slots=None) == PA_EINVAL
    assert call(T=-1) == PA_EINVAL
    assert call(Hkv=0) == PA_EINVAL
    assert call(D=12) == PA_EINVAL
    assert call(D=24) == PA_EINVAL
    assert call(ks=0.0) == PA_EINVAL
    assert call(vs=float("nan")) == PA_EINVAL
    assert call(k=ctypes.c_void_p(0x60008)) == PA_EALIGN
    bad = pa.PaKvPool(k_pool=0x10008, v_pool=0x20000, page_stride=256 * 16, token_stride=256,
                      head_stride=256, num_pages=8, page_size=16)
    assert call(kv=bad) == PA_EALIGN


@no_device
def test_cache_write_without_device_reports_edevice(L):
    pool = pa.PaKvPool(k_pool=0x10000, v_pool=0x20000, page_stride=256 * 16, token_stride=256,
                       head_stride=256, num_pages=8, page_size=16)
    A = ctypes.c_void_p(0x60000)
    assert L.paged_attn_cache_write_e4m3(A, A, 4, 1, 256, A, ctypes.byref(pool), 0.5, 2.0,
                                         None) == PA_EDEVICE


def test_combine_lse_rejects_bad_arguments(L):
    A = ctypes.c_void_p(0x10000)
    f = L.paged_attn_combine_fp32_lse
    assert f(A, A, A, 4, 48, 256, 1.0, None, None, None, None) == PA_EINVAL   # no output
    assert f(None, A, A, 4, 48, 256, 1.0, A, None, None, None) == PA_EINVAL
    assert f(A, A, A, 0, 48, 256, 1.0, A, None, None, None) == PA_EINVAL
    assert f(A, A, A, 4, 48, 254, 1.0, A, None, None, None) == PA_EINVAL
    assert f(A, A, A, 4, 48, 256, float("inf"), None, A, None, None) == PA_EINVAL
    assert f(A, A, A, 4, 48, 256, 1.0, None, ctypes.c_void_p(0x10008), None, None) == PA_EALIGN
    assert f(A, A, A, 4, 48, 256, 1.0, None, None, ctypes.c_void_p(0x10002), None) == PA_EALIGN
    assert f(A, A, A, 4, 48, 256, 1.0, ctypes.c_void_p(0x10004), None, None, None) == PA_EALIGN


@no_device
def test_combine_lse_without_device_reports_edevice(L):
    A = ctypes.c_void_p(0x10000)
    assert L.paged_attn_combine_fp32_lse(A, A, A, 4, 48, 256, 1.0, None, None, A, None) == PA_EDEVICE


def test_timer_rejects_bad_arguments(L):
    n = ctypes.c_int32(7)
    ms = (ctypes.c_float * 4)()
    assert L.paged_attn_timer_arm(-1) == PA_EINVAL
    assert L.paged_attn_timer_arm(pa.TIMER_MAX_LAUNCHES + 1) == PA_EINVAL
    assert L.paged_attn_timer_read(ms, 4, None) == PA_EINVAL
    assert L.paged_attn_timer_read(None, 4, ctypes.byref(n)) == PA_EINVAL
    assert L.paged_attn_timer_read(ms, -1, ctypes.byref(n)) == PA_EINVAL
    # nothing armed: nothing timed
    assert L.paged_attn_timer_read(None, 0, ctypes.byref(n)) == PA_OK and n.value == 0


def test_stream_read_probe_rejects_bad_arguments(L):
    A = ctypes.c_void_p(0x10000)
    assert L.paged_attn_stream_read_probe(None, 64, A, None) == PA_EINVAL
    assert L.paged_attn_stream_read_probe(A, 64, None, None) == PA_EINVAL
    assert L.paged_attn_stream_read_probe(A, -16, A, None) == PA_EINVAL
    assert L.paged_attn_stream_read_probe(A, 40, A, None) == PA_EINVAL
    assert L.paged_attn_stream_read_probe(ctypes.c_void_p(0x10008), 64, A, None) == PA_EALIGN


@no_device
def test_timer_without_device_reports_edevice(L):
    assert L.paged_attn_timer_arm(4) == PA_EDEVICE
    assert L.paged_attn_timer_arm(0) == PA_EDEVICE


def test_python_binding_rejects_cpu_fallback(monkeypatch, tmp_path):
    """Without the built library every op raises: there is no CPU path."""
    monkeypatch.setattr(pa, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(pa, "_LIB", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        pa.lib()


@pytest.mark.parametrize("cname,pyname", [("pa_plan", "PaPlan"), ("pa_workspace", "PaWorkspace"),
                                          ("pa_kv_pool", "PaKvPool")])
def test_struct_layout_matches_header(tmp_path, cname, pyname):
    """The binding's ctypes structs have the header's size and field offsets
    (a C program built against the header prints them)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    cls = getattr(pa, pyname)
    fields = [f[0] for f in cls._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'    printf("{f} %zu\\n", offsetof({cname}, {f}));\n' for f in fields)
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "paged_attn_e4m3.h"\n'
                   "int main(void) {\n"
                   f'    printf("sizeof %zu\\n", sizeof({cname}));\n{body}    return 0;\n}}\n')
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c11", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)],
                   check=True, capture_output=True)
    got = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                      text=True).stdout.splitlines())
    assert int(got["sizeof"]) == ctypes.sizeof(cls)
    for f in fields:
        assert int(got[f]) == getattr(cls, f).offset, f
