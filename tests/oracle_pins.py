"""Pins of the FP64 oracle against facts that do not come from the oracle.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
(or lets a precondition error escape) when the oracle disagrees with:
  * the E4M3 format definition (hand-derived spot values in
    tests/golden/e4m3_spot_values.txt) and PyTorch's float8_e4m3fn codec;
  * numpy's float16 and PyTorch's bfloat16 decoders;
  * PyTorch's scaled_dot_product_attention in float64 on the same tokens,
    gathered into an unpaged tensor by numpy indexing (the special case
    "one contiguous cache, plain softmax attention");
  * closed forms (one visible token, equal keys, constant values);
  * invariants (page relocation, NaN-poisoned masked bytes, zero-length
    rows, split-then-combine equal to one pass, selection order).

The same functions run against builds of the oracle with a planted mistake,
to show that every planted mistake fails at least one pin.
"""

from __future__ import annotations

import math
import os

import numpy as np
import torch

from fp8_kv_paged_attn_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Independent helpers (library decoders + SDPA)
# ---------------------------------------------------------------------------


def torch_e4m3(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_bf16(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def fp16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def sdpa_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, mask: np.ndarray,
              scale: float) -> np.ndarray:
    """Textbook attention with PyTorch: q [R][D], k/v [N][D], mask [R][N] (True = seen).

    Rows with no visible token give 0 (the reading for zero-length rows)."""
    R, D = q.shape
    out = np.zeros((R, D), np.float64)
    live = mask.any(axis=1)
    if live.any() and k.shape[0] > 0:
        qt = torch.from_numpy(q[live]).unsqueeze(0)
        kt = torch.from_numpy(np.ascontiguousarray(k)).unsqueeze(0)
        vt = torch.from_numpy(np.ascontiguousarray(v)).unsqueeze(0)
        mt = torch.from_numpy(mask[live]).unsqueeze(0)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt,
                                                             scale=scale)
        out[live] = o.squeeze(0).numpy()
    return out


def dense_reference(w) -> np.ndarray:
    """Library reference for a DenseWorkload: gather logical tokens, decode with
    PyTorch's float8_e4m3fn, repeat KV heads over their query-head groups, SDPA."""
    L = np.clip(w.row_lens.astype(np.int64), 0, w.max_tokens)
    n = int(L.max(initial=0))
    t = np.arange(n)
    phys = w.block_table.astype(np.int64)[t // w.page_size]
    k = torch_e4m3(w.k_pool[phys, t % w.page_size])        # [n][Hkv][D]
    v = torch_e4m3(w.v_pool[phys, t % w.page_size])
    G = w.num_heads // w.num_kv_heads
    q = fp16_bits_to_f64(w.q_bits)                         # [q][H][D]
    out = np.zeros(q.shape, np.float64)
    mask = t[None, :] < L[:, None]                         # [q][n]
    kr = np.repeat(k, G, axis=1)                           # head h uses kv head h // G
    vr = np.repeat(v, G, axis=1)
    for h in range(w.num_heads):
        out[:, h, :] = sdpa_rows(q[:, h, :], kr[:, h, :], vr[:, h, :], mask,
                                 w.sm_scale * w.k_scale)
    return out * w.v_scale


def qsa_reference(w) -> np.ndarray:
    """Library reference for a QsaWorkload: per (b, g) gather the selected blocks
    (a multiset), decode with PyTorch, mask t >= len, SDPA."""
    B, qr, H, D = w.q_bits.shape
    G = H // w.num_kv_heads
    q = torch_bf16(w.q_bits)
    out = np.zeros(q.shape, np.float64)
    cap = w.max_blocks * w.page_size
    for b in range(B):
        L = np.clip(w.row_lens[b].astype(np.int64), 0, cap)
        for g in range(w.num_kv_heads):
            blocks = [int(s) for s in w.sel_blocks[b, g] if s >= 0]
            if blocks:
                toks = np.concatenate([np.arange(s * w.page_size, (s + 1) * w.page_size)
                                       for s in blocks])
                phys = np.concatenate([np.full(w.page_size, w.block_table[b, s])
                                       for s in blocks]).astype(np.int64)
            else:
                toks = np.zeros(0, np.int64)
                phys = np.zeros(0, np.int64)
            u = toks % w.page_size
            k = torch_e4m3(w.k_pool[phys, u, g])
            v = torch_e4m3(w.v_pool[phys, u, g])
            mask = toks[None, :] < L[:, None]
            for h in range(g * G, (g + 1) * G):
                out[b, :, h, :] = sdpa_rows(q[b, :, h, :], k, v, mask, w.sm_scale * w.k_scale)
    return out * w.v_scale


def qsa_tokens_reference(w) -> np.ndarray:
    """Library reference for a QsaTokensWorkload: per (b, g) gather the selected
    token ids (a multiset, -1 skipped) through the block table, decode with
    PyTorch, mask id >= len per row, SDPA."""
    B, qr, H, D = w.q_bits.shape
    G = H // w.num_kv_heads
    q = torch_bf16(w.q_bits)
    out = np.zeros(q.shape, np.float64)
    cap = w.max_blocks * w.page_size
    for b in range(B):
        L = np.clip(w.row_lens[b].astype(np.int64), 0, cap)
        for g in range(w.num_kv_heads):
            toks = np.array([int(t) for t in w.sel_tokens[b, g] if 0 <= t < cap], np.int64)
            phys = w.block_table[b][toks // w.page_size].astype(np.int64)
            u = toks % w.page_size
            k = torch_e4m3(w.k_pool[phys, u, g])
            v = torch_e4m3(w.v_pool[phys, u, g])
            mask = toks[None, :] < L[:, None]
            for h in range(g * G, (g + 1) * G):
                out[b, :, h, :] = sdpa_rows(q[b, :, h, :], k, v, mask, w.sm_scale * w.k_scale)
    return out * w.v_scale


def assert_close_rel(a, b, rtol, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), f"{what}: non-finite"
    scale = max(float(np.abs(b).max(initial=0.0)), 1e-300)
    err = float(np.abs(a - b).max(initial=0.0))
    assert err <= rtol * scale, f"{what}: max err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _with_pool(w, k_pool, v_pool, block_table=None):
    import dataclasses

    kw = dict(k_pool=k_pool, v_pool=v_pool)
    if block_table is not None:
        kw["block_table"] = block_table
    return dataclasses.replace(w, **kw)


# ---------------------------------------------------------------------------
# Number-format pins
# ---------------------------------------------------------------------------


def pin_e4m3_golden(o):
    tab = o.e4m3_table()
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_spot_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, val = line.split()
            c = int(code, 16)
            exp = float(val)
            if math.isnan(exp):
                assert math.isnan(tab[c]), f"code {code} should be NaN"
            else:
                assert tab[c] == exp, f"code {code}: {tab[c]} != {exp}"
                assert math.copysign(1.0, tab[c]) == math.copysign(1.0, exp), f"sign of {code}"
            n += 1
    assert n >= 20


def pin_e4m3_vs_torch(o):
    tab = o.e4m3_table()
    ref = torch_e4m3(np.arange(256, dtype=np.uint8))
    same = (tab == ref) | (np.isnan(tab) & np.isnan(ref))
    assert same.all(), f"codes differ from float8_e4m3fn: {np.nonzero(~same)[0][:8]}"
    assert (np.signbit(tab) == np.signbit(ref))[~np.isnan(ref)].all()


def pin_e4m3_structure(o):
    tab = o.e4m3_table()
    assert int(np.isfinite(tab).sum()) == 254
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase"
    assert np.all(tab[0x80:0xFF] == -pos)
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9
    assert np.all(np.mod(pos * 512.0, 1.0) == 0.0), "every value is a multiple of 2^-9"


def pin_encoder_roundtrip(o):
    tab = o.e4m3_table()
    codes = np.array([c for c in range(256) if np.isfinite(tab[c])], np.uint8)
    got = o.e4m3_encode(tab[codes])
    assert np.array_equal(got, codes), "encode(decode(c)) != c"


def _encoder_sweep() -> np.ndarray:
    tab = torch_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (tab[:-1] + tab[1:]) / 2.0
    m32 = mids.astype(np.float32)
    pts = [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1000)),
           tab.astype(np.float32),
           np.linspace(0.0, 463.9, 20001, dtype=np.float32),
           np.float32(2.0) ** np.arange(-14, 9, 0.125, dtype=np.float32)]
    x = np.concatenate(pts).astype(np.float32)
    x = x[np.abs(x) < 464.0]
    return np.concatenate([x, -x])


def pin_encoder_vs_torch(o):
    x = _encoder_sweep()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = o.e4m3_encode(x.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"encoder differs at {x[bad[:5]]}: {got[bad[:5]]} vs {ref[bad[:5]]}"
    sat = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e4, np.inf])
    assert np.all(o.e4m3_encode(sat) == 0x7E)
    assert np.all(o.e4m3_encode(-sat) == 0xFE)
    assert o.e4m3_encode([np.nan])[0] == 0x7F
    assert o.e4m3_encode([-0.0])[0] == 0x80 and o.e4m3_encode([2.0 ** -10])[0] == 0x00


def pin_fp16_decode(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    step = 97 if os.environ.get("ORC_PIN_QUICK") else 1
    for b in range(0, 65536, step):
        got = o.fp16_value(b)
        r = ref[b]
        assert (got == r) or (math.isnan(got) and math.isnan(r)), f"fp16 {b:#06x}: {got} vs {r}"


def pin_bf16_decode(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch_bf16(bits)
    step = 97 if os.environ.get("ORC_PIN_QUICK") else 1
    for b in range(0, 65536, step):
        got = o.bf16_value(b)
        r = ref[b]
        assert (got == r) or (math.isnan(got) and math.isnan(r)), f"bf16 {b:#06x}: {got} vs {r}"


# ---------------------------------------------------------------------------
# Attention pins
# ---------------------------------------------------------------------------

_DENSE_CASES = [
    dict(q_rows=2, num_heads=4, num_kv_heads=2, head_dim=16, ctx=37, page_size=5,
         pool_pages=12, row_lens=[36, 37]),
    dict(q_rows=3, num_heads=6, num_kv_heads=1, head_dim=32, ctx=50, page_size=7,
         pool_pages=9, row_lens=[0, 23, 50]),
    dict(q_rows=1, num_heads=2, num_kv_heads=2, head_dim=8, ctx=6, page_size=1,
         pool_pages=8, row_lens=[6]),
    dict(q_rows=4, num_heads=8, num_kv_heads=4, head_dim=16, ctx=41, page_size=16,
         pool_pages=5, row_lens=[-3, 41, 99, 17]),
    dict(q_rows=2, num_heads=6, num_kv_heads=1, head_dim=64, ctx=130, page_size=48,
         pool_pages=6, row_lens=[129, 130]),
]


def _dense_case(i, **over):
    kw = dict(_DENSE_CASES[i])
    kw.update(over)
    return wl.make_dense(f"pin{i}", 0xA11CE + i, sigma=1.3, k_scale=0.6, v_scale=1.7,
                         **kw)


def pin_dense_vs_sdpa(o):
    for i in range(len(_DENSE_CASES)):
        w = _dense_case(i)
        got = o.dense_workload(w)
        ref = dense_reference(w)
        assert_close_rel(got, ref, 1e-12, f"dense case {i}")


def _qsa_case(seed, **over):
    kw = dict(batch=2, q_rows=2, num_heads=4, num_kv_heads=2, head_dim=16, ctx=64,
              page_size=8, topk=4, k_scale=0.5, v_scale=2.0)
    kw.update(over)
    return wl.make_qsa(f"pinqsa{seed}", seed, **kw)


def pin_qsa_vs_sdpa(o):
    import dataclasses

    w = _qsa_case(0xB0B)
    assert_close_rel(o.qsa_workload(w), qsa_reference(w), 1e-12, "qsa basic")
    # empty slots, a duplicated block, and a length that cuts the newest block
    sel = w.sel_blocks.copy()
    sel[0, 0, 1] = -1
    sel[1, 1, 0] = sel[1, 1, 2]
    lens = w.row_lens.copy()
    lens[0, 0] = 61
    lens[1, 1] = 0
    w2 = dataclasses.replace(w, sel_blocks=sel, row_lens=lens)
    assert_close_rel(o.qsa_workload(w2), qsa_reference(w2), 1e-12, "qsa edge")
    w3 = _qsa_case(0xB0C, num_heads=6, num_kv_heads=3, head_dim=32, q_rows=3, topk=3)
    assert_close_rel(o.qsa_workload(w3), qsa_reference(w3), 1e-12, "qsa G2")


def pin_closed_forms(o):
    import dataclasses

    w = _dense_case(4)
    tab = o.e4m3_table()
    # one visible token: output = v_scale * v(token 0), exactly
    w1 = dataclasses.replace(w, row_lens=np.array([1, 1], np.int32))
    got = o.dense_workload(w1)
    p0 = int(w.block_table[0])
    v0 = tab[w.v_pool[p0, 0, 0]]
    assert np.array_equal(got[0, 0], w.v_scale * v0), "one-token row"
    # all keys equal: output = v_scale * mean of the visible values
    k = w.k_pool.copy()
    k[...] = w.k_pool[p0, 0, 0][None, None, None, :]
    w2 = _with_pool(w, k, w.v_pool)
    got = o.dense_workload(w2)
    n = int(w.row_lens[0])
    t = np.arange(n)
    vv = tab[w.v_pool[w.block_table[t // w.page_size], t % w.page_size, 0]]
    assert_close_rel(got[0, 3], w.v_scale * vv.mean(axis=0), 1e-13, "equal keys")
    # constant V = c: output = v_scale * c
    v = np.full_like(w.v_pool, 0x3A)        # 1.25
    w3 = _with_pool(w, w.k_pool, v)
    got = o.dense_workload(w3)
    assert np.allclose(got, w.v_scale * 1.25, rtol=1e-14, atol=0), "constant V"
    # k_scale tiny: softmax -> uniform average
    w4 = dataclasses.replace(w, k_scale=1e-30)
    got = o.dense_workload(w4)
    assert_close_rel(got[1, 5], w.v_scale * tab[w.v_pool[w.block_table[
        np.arange(130) // 48], np.arange(130) % 48, 0]].mean(axis=0), 1e-12, "tiny k_scale")


def pin_one_hot_probe(o):
    """K = 448 on one token, 0 elsewhere, q all ones: the softmax is one-hot in
    FP64, so the output equals v_scale * V(probe) exactly, for probes at page
    starts, page ends and in the partial last page, under relocation."""
    import dataclasses

    base = _dense_case(4)
    tab = o.e4m3_table()
    ones = np.full(base.q_bits.shape, np.float16(1.0)).view(np.uint16)
    for probe in [0, 47, 48, 95, 96, 129, 128]:
        k = np.zeros_like(base.k_pool)
        lp, u = divmod(probe, base.page_size)
        p = int(base.block_table[lp])
        k[p, u, 0, :] = 0x7E
        w = dataclasses.replace(base, k_pool=k, q_bits=ones, k_scale=1.0,
                                row_lens=np.array([130, 130], np.int32))
        got = o.dense_workload(w)
        exp = w.v_scale * tab[base.v_pool[p, u, 0]]
        assert np.array_equal(got[0, 2], exp) and np.array_equal(got[1, 5], exp), \
            f"probe token {probe}"


def pin_relocation(o):
    """Moving pages to other physical slots (and rewriting the table) leaves the
    output bit-identical."""
    w = _dense_case(0)
    P = w.k_pool.shape[0]
    perm = np.roll(np.arange(P), 5)                       # physical p -> perm[p]
    k = np.empty_like(w.k_pool)
    v = np.empty_like(w.v_pool)
    k[perm] = w.k_pool
    v[perm] = w.v_pool
    w2 = _with_pool(w, k, v, perm[w.block_table].astype(np.int32))
    assert np.array_equal(o.dense_workload(w), o.dense_workload(w2)), "dense relocation"
    q = _qsa_case(0xB0D)
    P = q.k_pool.shape[0]
    perm = np.roll(np.arange(P), 3)
    k = np.empty_like(q.k_pool)
    v = np.empty_like(q.v_pool)
    k[perm] = q.k_pool
    v[perm] = q.v_pool
    q2 = _with_pool(q, k, v, perm[q.block_table].astype(np.int32))
    assert np.array_equal(o.qsa_workload(q), o.qsa_workload(q2)), "qsa relocation"


def pin_nan_poison(o):
    """NaN bytes at masked positions (tail of the last page, padded table entries
    pointing at a NaN null page, unselected pages) leave the output identical;
    zero-length rows give exactly 0."""
    import dataclasses

    w = wl.make_dense("poison", 0xBAD, q_rows=3, num_heads=4, num_kv_heads=2,
                      head_dim=16, ctx=40, page_size=16, pool_pages=6, sigma=1.0,
                      k_scale=0.5, v_scale=2.0, row_lens=[0, 39, 40],
                      null_page_nan=False, poison_unused=False)
    clean = o.dense_workload(w)
    assert np.all(np.isfinite(clean))
    assert np.array_equal(clean[0], np.zeros_like(clean[0])), "zero-length row"
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    used = set(int(p) for p in w.block_table)
    for p in range(k.shape[0]):
        if p not in used:
            k[p] = 0x7F
            v[p] = 0xFF
    last = int(w.block_table[-1])
    k[last, 40 - 32:] = 0x7F
    v[last, 40 - 32:] = 0x7F
    table = np.concatenate([w.block_table, [p for p in range(k.shape[0]) if p not in used][:2]])
    w2 = _with_pool(w, k, v, table.astype(np.int32))
    assert np.array_equal(o.dense_workload(w2), clean), "poisoned masked bytes changed output"
    q = _qsa_case(0xBAE)
    assert np.all(np.isfinite(o.qsa_workload(q))), "qsa with NaN unselected pages"
    lens = q.row_lens.copy()
    lens[1, 0] = 0
    qz = dataclasses.replace(q, row_lens=lens)
    assert np.array_equal(o.qsa_workload(qz)[1, 0], np.zeros((4, 16))), "qsa zero row"


def pin_visible_nan(o):
    """NaN bytes at positions a row sees: a NaN K byte makes every row seeing
    the token NaN, a NaN V byte makes that column NaN for the rows seeing it
    (PyTorch SDPA on the decoded tokens agrees); split partials combined give
    the same NaN pattern and the same finite values as the one-pass result."""
    w = _dense_case(1)                       # H6/Hkv1/D32, page 7, lengths 0, 23, 50
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    tk, tv, dv = 30, 10, 5                   # token 30: row 2 only; token 10: rows 1, 2
    k[w.block_table[tk // w.page_size], tk % w.page_size, 0, 3] = 0x7F
    v[w.block_table[tv // w.page_size], tv % w.page_size, 0, dv] = 0xFF
    w2 = _with_pool(w, k, v)
    one = o.dense_workload(w2)
    assert np.all(np.isnan(one[2])), "row seeing the NaN key"
    assert np.all(np.isnan(one[1][:, dv])), "column of the NaN value"
    assert np.all(np.isfinite(np.delete(one[1], dv, axis=1)))
    assert not one[0].any(), "zero-length row"
    # SDPA per row over that row's visible tokens only (a boolean mask is
    # additive inside SDPA, so a NaN key it masks would still reach the row)
    q = fp16_bits_to_f64(w2.q_bits)
    t = np.arange(w2.max_tokens)
    phys = w2.block_table[t // w2.page_size]
    kd = torch_e4m3(w2.k_pool[phys, t % w2.page_size, 0])
    vd = torch_e4m3(w2.v_pool[phys, t % w2.page_size, 0])
    ref = np.zeros_like(one)
    for i, L in enumerate(w2.row_lens):
        if L > 0:
            ref[i] = sdpa_rows(q[i], kd[:L], vd[:L], np.ones((w2.num_heads, L), bool),
                               w2.sm_scale * w2.k_scale) * w2.v_scale
    assert np.array_equal(np.isnan(ref), np.isnan(one)), "NaN pattern vs SDPA"
    fin = np.isfinite(one)
    assert_close_rel(one[fin], ref[fin], 1e-12, "finite part vs SDPA")
    for S, T in [(1, 64), (4, 13), (7, 8), (60, 1)]:
        acc, mx, sm = o.verify_dense_split(w2.q_bits, w2.k_pool, w2.v_pool, w2.block_table,
                                           w2.row_lens, w2.max_tokens, w2.num_kv_heads,
                                           w2.sm_scale, w2.k_scale, S, T)
        comb = o.combine(acc, mx, sm, w2.v_scale).reshape(one.shape)
        assert np.array_equal(np.isnan(comb), np.isnan(one)), f"NaN pattern S={S}"
        assert_close_rel(comb[fin], one[fin], 1e-12, f"finite part S={S}")


def pin_split_combine(o):
    """Split partials combined give the one-pass result (<= 1e-12 relative) for
    S in {1, 2, 4, 7, many}, including splits past every length; each split's
    base-2 LSE matches torch.logsumexp and its normalised numerator matches
    SDPA over that split's tokens."""
    w = _dense_case(1)                       # lengths 0, 23, 50
    one = o.dense_workload(w)
    R = w.q_rows * w.num_heads
    for S, T in [(1, 64), (2, 25), (4, 13), (7, 8), (60, 1), (9, 16)]:
        acc, mx, sm = o.verify_dense_split(w.q_bits, w.k_pool, w.v_pool, w.block_table,
                                           w.row_lens, w.max_tokens, w.num_kv_heads,
                                           w.sm_scale, w.k_scale, S, T)
        comb = o.combine(acc, mx, sm, w.v_scale).reshape(one.shape)
        assert_close_rel(comb, one, 1e-12, f"split S={S} T={T}")
        # per-split checks on row (i=2, h=1)
        i, h = 2, 1
        row = i * w.num_heads + h
        q = fp16_bits_to_f64(w.q_bits)[i, h]
        t = np.arange(50)
        phys = w.block_table[t // w.page_size]
        k = torch_e4m3(w.k_pool[phys, t % w.page_size, 0])
        v = torch_e4m3(w.v_pool[phys, t % w.page_size, 0])
        s = (k @ q) * (w.sm_scale * w.k_scale)
        for sp in range(S):
            lo, hi = sp * T, min((sp + 1) * T, 50)
            if lo >= hi:
                assert mx[sp, row] == -np.inf and sm[sp, row] == 0.0
                assert not acc[sp, row].any()
                continue
            lse = float(torch.logsumexp(torch.from_numpy(s[lo:hi]), 0)) / math.log(2.0)
            got = mx[sp, row] + math.log2(sm[sp, row])
            assert abs(got - lse) <= 1e-12 * max(1.0, abs(lse)), f"split {sp} LSE"
            ref = sdpa_rows(q[None], k[lo:hi], v[lo:hi], np.ones((1, hi - lo), bool),
                            w.sm_scale * w.k_scale)[0]
            assert_close_rel(acc[sp, row] / sm[sp, row], ref, 1e-12, f"split {sp} numerator")
    # zero-length row: every split empty
    acc, mx, sm = o.verify_dense_split(w.q_bits, w.k_pool, w.v_pool, w.block_table,
                                       w.row_lens, w.max_tokens, w.num_kv_heads,
                                       w.sm_scale, w.k_scale, 4, 13)
    assert np.all(mx[:, :w.num_heads] == -np.inf) and not sm[:, :w.num_heads].any()
    # QSA split by list position
    q = _qsa_case(0xB0E)
    oneq = o.qsa_workload(q)
    for S, T in [(1, 32), (4, 8), (3, 11), (40, 1)]:
        acc, mx, sm = o.qsa_split(q.q_bits, q.k_pool, q.v_pool, q.block_table, q.sel_blocks,
                                  q.row_lens, q.sm_scale, q.k_scale, S, T)
        comb = o.combine(acc, mx, sm, q.v_scale).reshape(oneq.shape)
        assert_close_rel(comb, oneq, 1e-12, f"qsa split S={S}")


def lse_merge(parts):
    """Merge (out, lse) pairs of disjoint token sets of the same rows:
    LSE = log2 sum_k 2^lse_k, o = sum_k 2^(lse_k - LSE) o_k; rows empty in every
    part give 0."""
    lses = np.stack([l for _, l in parts])
    top = lses.max(axis=0)
    safe = np.where(np.isfinite(top), top, 0.0)
    w = np.exp2(lses - safe)                                  # 0 for empty parts
    tot = w.sum(axis=0)
    out = sum(wk[:, None] * ok for wk, (ok, _) in zip(w, parts))
    out = np.where(tot[:, None] > 0, out / np.where(tot > 0, tot, 1.0)[:, None], 0.0)
    return out, np.where(tot > 0, safe + np.log2(np.where(tot > 0, tot, 1.0)), -np.inf)


def pin_combine_lse(o):
    """The base-2 LSE of a row is log2 sum_t 2^(y_t), i.e. torch.logsumexp of its
    logits over ln 2 (-inf for an empty row), and two disjoint groups of splits,
    each combined with its LSE and then merged by the LSE rule, give the one-pass
    output and LSE."""
    w = _dense_case(1)                       # H6/Hkv1/D32, page 7, lengths 0, 23, 50
    S, T = 7, 8
    acc, mx, sm = o.verify_dense_split(w.q_bits, w.k_pool, w.v_pool, w.block_table,
                                       w.row_lens, w.max_tokens, w.num_kv_heads,
                                       w.sm_scale, w.k_scale, S, T)
    out, lse = o.combine(acc, mx, sm, w.v_scale, with_lse=True)
    assert np.array_equal(out, o.combine(acc, mx, sm, w.v_scale)), "lse form changes out"
    q = fp16_bits_to_f64(w.q_bits)
    t = np.arange(w.max_tokens)
    k = torch_e4m3(w.k_pool[w.block_table[t // w.page_size], t % w.page_size, 0])
    for i, L in enumerate(w.row_lens):
        for h in range(w.num_heads):
            r = i * w.num_heads + h
            if L <= 0:
                assert lse[r] == -np.inf, "empty row"
                continue
            s = (k[:L] @ q[i, h]) * (w.sm_scale * w.k_scale)
            ref = float(torch.logsumexp(torch.from_numpy(s), 0)) / math.log(2.0)
            assert abs(lse[r] - ref) <= 1e-12 * max(1.0, abs(ref)), f"lse row {r}"
    for cut in (1, 3, 6):
        a = o.combine(acc[:cut], mx[:cut], sm[:cut], w.v_scale, with_lse=True)
        b = o.combine(acc[cut:], mx[cut:], sm[cut:], w.v_scale, with_lse=True)
        mo, ml = lse_merge([a, b])
        assert_close_rel(mo, out, 1e-12, f"merged output, cut {cut}")
        live = np.isfinite(lse)
        assert np.array_equal(np.isfinite(ml), live)
        assert_close_rel(ml[live], lse[live], 1e-12, f"merged lse, cut {cut}")


def _f32_partials_with_specials(seed: int, S: int, R: int, D: int):
    """FP32 split partials as a verify kernel writes them, plus the cases a
    combine must handle: empty splits (sum 0) whose max and numerator hold
    garbage (-inf, NaN, inf), a NaN sum with a -inf max, a NaN in a numerator
    of a non-empty split, and rows whose every split is empty."""
    rng = np.random.default_rng(seed)
    mx = rng.normal(0.0, 6.0, (S, R)).astype(np.float32)
    sm = rng.uniform(0.5, 40.0, (S, R)).astype(np.float32)
    acc = (rng.normal(0.0, 3.0, (S, R, D)) * sm[:, :, None]).astype(np.float32)
    empty = rng.random((S, R)) < 0.2
    sm[empty] = 0.0
    mx[empty] = rng.choice(np.array([-np.inf, np.nan, np.inf, 7.0], np.float32), empty.sum())
    acc[empty] = np.nan
    sm[:, 0] = 0.0                                   # row 0: every split empty
    mx[:, 0] = -np.inf
    sm[1, 1], mx[1, 1] = np.nan, -np.inf             # NaN sum reaches row 1
    sm[2, 2] = 3.0
    acc[2, 2, 3] = np.nan                            # NaN numerator, column 3 of row 2
    return acc, mx, sm


def pin_combine_f32(o):
    """The combine of FP32 partials (the form a GPU workspace holds, used to
    check the combine kernel) equals, bit for bit, the combine of the same
    values converted to FP64, which the other pins tie to the one-pass
    definition and to logsumexp: with and without the LSE, on real split
    partials rounded to FP32 and on random partials with empty splits full of
    garbage, NaN sums and NaN numerators.  Real partials rounded to FP32 also
    combine to the one-pass FP64 output within FP32 rounding."""
    w = _dense_case(1)                               # lengths 0, 23, 50
    one = o.dense_workload(w)
    acc, mx, sm = o.verify_dense_split(w.q_bits, w.k_pool, w.v_pool, w.block_table,
                                       w.row_lens, w.max_tokens, w.num_kv_heads,
                                       w.sm_scale, w.k_scale, 7, 8)
    cases = [tuple(x.astype(np.float32) for x in (acc, mx, sm)),
             _f32_partials_with_specials(0xC0B32, 37, 12, 16)]
    for n, (a32, m32, s32) in enumerate(cases):
        a64, m64, s64 = (x.astype(np.float64) for x in (a32, m32, s32))
        for vs in (1.0, 2.25):
            got = o.combine(a32, m32, s32, vs)
            ref = o.combine(a64, m64, s64, vs)
            assert np.array_equal(got, ref, equal_nan=True), f"fp32 combine, case {n}"
            go, gl = o.combine(a32, m32, s32, vs, with_lse=True)
            ro, rl = o.combine(a64, m64, s64, vs, with_lse=True)
            assert np.array_equal(go, ref, equal_nan=True), f"fp32 lse combine out, case {n}"
            assert np.array_equal(gl, rl, equal_nan=True), f"fp32 lse, case {n}"
    a32, m32, s32 = cases[0]
    got = o.combine(a32, m32, s32, w.v_scale).reshape(one.shape)
    assert_close_rel(got, one, 4e-7, "fp32 partials against the one-pass output")
    a32, m32, s32 = cases[1]
    got = o.combine(a32, m32, s32, 1.0)
    assert not got[0].any(), "row with every split empty"
    assert np.isnan(got[1]).all(), "NaN sum reaches its row"
    assert np.isnan(got[2, 3]) and np.isfinite(np.delete(got[2], 3)).all(), "NaN numerator"
    assert np.isfinite(got[3:]).all(), "garbage in empty splits leaked"


def pin_cache_write(o):
    """The cache write puts E4M3(fp32(x) / fp32(scale)) at each slot's bytes and
    touches nothing else: PyTorch's float8_e4m3fn cast of the same FP32 quotient
    gives the same code below 448, saturation gives 0x7E at and above it, NaN
    gives 0x7F, -0 gives 0x80, and ties go to the even code."""
    rng = np.random.Generator(np.random.PCG64(0xCAC4E))
    T, Hkv, D, P, ps = 37, 2, 16, 6, 8
    vals = rng.standard_normal((T, Hkv, D)) * np.array([0.3, 40.0])[None, :, None]
    vals = vals.astype(np.float16)
    vals[0, 0, :6] = [0.0, -0.0, np.nan, np.inf, -np.inf, 60000.0]
    vals[1, 0, :4] = [1.0625, 1.1875, -1.0625, 2 ** -10]      # ties, and a subnormal half-step
    k_bits = vals.view(np.uint16)
    v_bits = (-vals).view(np.uint16)
    slots = rng.permutation(P * ps)[:T].astype(np.int64)
    slots[[5, 11]] = -1
    k0 = rng.integers(0, 256, (P, ps, Hkv, D), dtype=np.uint8)
    v0 = rng.integers(0, 256, (P, ps, Hkv, D), dtype=np.uint8)
    ks, vs = np.float32(0.5), np.float32(1.0)
    kp, vp = o.cache_write(k_bits, v_bits, slots, k0, v0, ks, vs)
    written = np.zeros((P, ps), bool)
    for t, sl in enumerate(slots):
        if sl >= 0:
            written[sl // ps, sl % ps] = True
    assert np.array_equal(kp[~written], k0[~written]) and np.array_equal(vp[~written], v0[~written])
    for plane, bits, scale in ((kp, k_bits, ks), (vp, v_bits, vs)):
        x = torch.from_numpy(bits.view(np.float16).astype(np.float32)) / float(scale)
        ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        xa = x.numpy()
        for t, sl in enumerate(slots):
            if sl < 0:
                continue
            got = plane[sl // ps, sl % ps]
            fin = np.isfinite(xa[t]) & (np.abs(xa[t]) < 448)
            assert np.array_equal(got[fin], ref[t][fin]), f"token {t} vs torch"
            sat = np.abs(xa[t]) >= 448
            assert np.all(got[sat] == (0x7E | np.where(xa[t][sat] < 0, 0x80, 0))), f"token {t} sat"
            assert np.all(got[np.isnan(xa[t])] == 0x7F), f"token {t} nan"
    # specials of token 0 (K plane, scale 0.5) and the ties of token 1
    k_tok = lambda t: kp[slots[t] // ps, slots[t] % ps, 0]
    assert list(k_tok(0)[:6]) == [0x00, 0x80, 0x7F, 0x7E, 0xFE, 0x7E]
    # x/0.5: 2.125 -> tie of 2.0 / 2.25 -> 2.0 (0x40); 2.375 -> tie of 2.25 / 2.5 -> 2.5 (0x42);
    # -2.125 -> 0xC0; 2^-9 (exactly the smallest subnormal) -> 0x01
    assert list(k_tok(1)[:4]) == [0x40, 0x42, 0xC0, 0x01]


def pin_selection_order(o):
    import dataclasses

    q = _qsa_case(0xB0F)
    base = o.qsa_workload(q)
    sel = q.sel_blocks[:, :, ::-1].copy()
    assert_close_rel(o.qsa_workload(dataclasses.replace(q, sel_blocks=sel)), base, 1e-13,
                     "reversed selection")
    # every block selected: any order of the same multiset gives the same output
    qd = _qsa_case(0xC0F, batch=1, num_kv_heads=1, num_heads=3, topk=8, ctx=64)
    shuffled = o.qsa_workload(qd)
    inorder = np.sort(qd.sel_blocks, axis=2)
    assert not np.array_equal(inorder, qd.sel_blocks)
    got = o.qsa_workload(dataclasses.replace(qd, sel_blocks=inorder))
    assert_close_rel(got, shuffled, 1e-13, "sorted selection")
    assert_close_rel(got, qsa_reference(qd), 1e-12, "all blocks selected")


def _tokens_case(seed, **over):
    kw = dict(batch=2, q_rows=3, num_heads=4, num_kv_heads=2, head_dim=16, ctx=100,
              page_size=16, num_sel=20, num_empty=3, k_scale=0.5, v_scale=2.0)
    kw.update(over)
    return wl.make_qsa_tokens(f"pintok{seed}", seed, **kw)


def pin_qsa_tokens(o):
    """Token-id selection: (1) a block selection written out as its token ids
    gives bit-for-bit the block-selection result, one pass and split (NaN
    bytes in every unselected page); (2) against SDPA over the selected ids
    with a per-row mask, including a duplicated id, a zero-length row, a row
    past the table and an id past the table; (3) split partials combined give
    the one-pass result."""
    import dataclasses

    q = _qsa_case(0xB10)
    tok = wl.tokens_from_blocks(q)
    one = o.qsa_tokens_verify(q.q_bits, q.k_pool, q.v_pool, q.block_table, tok, q.row_lens,
                              q.sm_scale, q.k_scale, q.v_scale)
    assert np.all(np.isfinite(one)), "token ids reached a poisoned page"
    assert np.array_equal(one, o.qsa_workload(q)), "token ids of a block selection"
    for S, T in [(3, 11), (8, 4)]:
        a = o.qsa_tokens_split(q.q_bits, q.k_pool, q.v_pool, q.block_table, tok, q.row_lens,
                               q.sm_scale, q.k_scale, S, T)
        b = o.qsa_split(q.q_bits, q.k_pool, q.v_pool, q.block_table, q.sel_blocks,
                        q.row_lens, q.sm_scale, q.k_scale, S, T)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), f"token-id split S={S}"

    w = _tokens_case(0xB11)
    assert_close_rel(o.qsa_tokens_workload(w), qsa_tokens_reference(w), 1e-12, "tokens basic")
    sel = w.sel_tokens.copy()
    sel[0, 1, 4] = sel[0, 1, 7]                  # a duplicated id counts twice
    sel[1, 0, 2] = 7 * w.page_size + 3           # id past the table: never seen
    lens = w.row_lens.copy()
    lens[0, 1] = 0
    lens[1, 2] = 10 ** 6                         # clamped to the table's capacity
    w2 = dataclasses.replace(w, sel_tokens=sel, row_lens=lens)
    got = o.qsa_tokens_workload(w2)
    assert_close_rel(got, qsa_tokens_reference(w2), 1e-12, "tokens edge")
    assert not got[0, 1].any(), "zero-length row"
    R = w2.num_rows
    for S, T in [(1, 20), (4, 5), (3, 7), (25, 1)]:
        acc, mx, sm = o.qsa_tokens_split(w2.q_bits, w2.k_pool, w2.v_pool, w2.block_table,
                                         w2.sel_tokens, w2.row_lens, w2.sm_scale,
                                         w2.k_scale, S, T)
        assert acc.shape == (S, R, w2.head_dim)
        comb = o.combine(acc, mx, sm, w2.v_scale).reshape(got.shape)
        assert_close_rel(comb, got, 1e-12, f"tokens split S={S}")


# Cheap pins first: the planted-mistake test stops at the first failure.
ALL_PINS = [
    pin_e4m3_golden, pin_e4m3_structure, pin_e4m3_vs_torch, pin_encoder_roundtrip,
    pin_encoder_vs_torch, pin_one_hot_probe, pin_closed_forms, pin_relocation,
    pin_nan_poison, pin_dense_vs_sdpa, pin_qsa_vs_sdpa, pin_split_combine, pin_visible_nan,
    pin_combine_lse, pin_combine_f32, pin_cache_write, pin_qsa_tokens,
    pin_selection_order, pin_fp16_decode, pin_bf16_decode,
]
