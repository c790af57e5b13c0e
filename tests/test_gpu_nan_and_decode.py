"""GPU tests through the C ABI: NaN bytes that some rows of a KV unit see and
others do not (the draft tokens of a causal verify), and every E4M3 code
through each decoder of both kernels.

NaN at a position a row sees is not specified by the pages; the reading here
is the plain definition (the oracle's): a NaN V byte makes that column NaN in
exactly the rows that see its token, a NaN K byte makes those rows NaN, and
every other output matches the oracle at the usual bar.  The pages' own rule
(1Cat-vLLM PR "Qualify calibrated E4M3 and disk PLE with QSA DCP2", null-block
fix: rows no query attends must not reach P.V) is the special case of a token
no row sees.

The decode checks use outputs the kernels produce exactly:
  * V: a one-hot softmax (K = 448 on one token, 0 elsewhere, q = 1) returns the
    probe token's V row, whose 256 bytes hold all 254 finite codes, as
    fp16(decode(code)) bit for bit (v_scale = 1);
  * K: with q = e_0 every score is K[t][0] exactly, and a split whose tokens
    all hold one code writes the split maximum fp32(decode(code) * c), c the
    folded logit scale, bit for bit; one split per code covers all 254.
"""

import dataclasses

import numpy as np
import pytest
import torch

import fp8_kv_paged_attn_amd as pa
from fp8_kv_paged_attn_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

KERNELS = ["mfma", "simple"]
FINITE_CODES = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)   # 254
LOG2E = 1.4426950408889634


def announce(*what):
    print("[case]", *what, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()


def assert_nan_parity(got, ref, what):
    got = np.asarray(got, np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern differs"
    fin = np.isfinite(ref)
    gu.assert_parity(got[fin], ref[fin], what)


def folded_scale(sm_scale, k_scale) -> np.float32:
    """The logit scale as the library folds it: fp32(sm * k * log2(e))."""
    return np.float32(np.float64(np.float32(sm_scale)) * np.float64(np.float32(k_scale)) * LOG2E)


# ---------------------------------------------------------------------------
# NaN bytes at positions some rows see
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_dense_nan_at_draft_tokens(orc, kernel, splits):
    """Causal verify of 8 rows: a NaN V byte at the first draft token (seen by
    rows 1-7, not row 0), a NaN K byte at a later draft token (rows 4-7) and a
    NaN V byte that every row sees: each output is NaN exactly where the oracle
    has NaN and matches it elsewhere, for one split, five and the planner's."""
    w = wl.make_dense("draftnan", 0xD4A, q_rows=8, num_heads=6, num_kv_heads=1, head_dim=256,
                      ctx=3000, page_size=848, pool_pages=6, sigma=1.0, k_scale=0.5,
                      v_scale=1.5, num_splits=splits)
    L = [int(x) for x in w.row_lens]
    assert L == [3000 - 8 + i + 1 for i in range(8)]
    k, v = w.k_pool.copy(), w.v_pool.copy()
    at = lambda t: (w.block_table[t // w.page_size], t % w.page_size, 0)
    v[at(L[0])][9] = 0x7F              # column 9 of rows 1-7
    k[at(L[0] + 3)][17] = 0xFF         # rows 4-7 entirely
    v[at(L[0] - 40)][200] = 0xFF       # column 200 of every row
    w = dataclasses.replace(w, k_pool=k, v_pool=v)
    announce("dense draft nan", kernel, splits)
    ref = orc.dense_workload(w)
    assert np.isnan(ref[4:]).all() and np.isnan(ref[1:4, :, 9]).all()
    assert np.isnan(ref[:4, :, 200]).all()
    assert np.isfinite(np.delete(ref[0], 200, axis=1)).all()
    assert_nan_parity(gu.run_dense(w, kernel), ref, f"dense draft nan/{kernel}/S{splits}")


def _sparse_case(seed):
    w = wl.make_qsa("qsanan", seed, batch=2, q_rows=4, num_heads=12, num_kv_heads=2,
                    head_dim=128, ctx=2048, page_size=64, topk=8, k_scale=0.5, v_scale=2.0,
                    num_splits=3)
    L = [int(x) for x in w.row_lens[0]]
    assert L == sorted(L) and L[0] < L[-1] <= 2048
    k, v = w.k_pool.copy(), w.v_pool.copy()
    at = lambda t, g: (w.block_table[0, t // w.page_size], t % w.page_size, g)
    v[at(L[0], 0)][5] = 0x7F           # request 0, KV head 0: column 5 of rows 1-3
    k[at(L[2], 1)][40] = 0x7F          # request 0, KV head 1: row 3 entirely
    return dataclasses.replace(w, k_pool=k, v_pool=v)


@pytest.mark.parametrize("kernel", KERNELS)
def test_sparse_nan_at_draft_tokens(orc, kernel):
    """The same in the newest selected block of the sparse path, over the block
    selection and over the same selection written as token ids."""
    w = _sparse_case(0x5A7)
    ref = orc.qsa_workload(w)
    assert np.isnan(ref[0, 1:, :6, 5]).all() and np.isfinite(ref[0, 0, :6]).all()
    assert np.isnan(ref[0, 3, 6:]).all() and np.isfinite(ref[0, :3, 6:]).all()
    assert np.isfinite(ref[1]).all()
    announce("sparse draft nan", kernel)
    assert_nan_parity(gu.run_qsa(w, kernel), ref, f"qsa draft nan/{kernel}")
    tok = wl.tokens_from_blocks(w)
    q = gu.bf16_tensor(w.q_bits).to(gu.DEV)
    kp = torch.from_numpy(w.k_pool).to(gu.DEV)
    vp = torch.from_numpy(w.v_pool).to(gu.DEV)
    bt = torch.from_numpy(w.block_table.astype(np.int32)).to(gu.DEV)
    sel = torch.from_numpy(tok.astype(np.int32)).to(gu.DEV)
    lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(gu.DEV)
    p = pa.plan(tok.shape[2], w.q_rows * (w.num_heads // w.num_kv_heads),
                w.batch * w.num_kv_heads, w.head_dim, w.page_size, "tokens", splits=3,
                kernel=kernel)
    got = pa.qsa_verify_tokens(q, kp, vp, bt, sel, lens, sm_scale=w.sm_scale,
                               k_scale=w.k_scale, v_scale=w.v_scale, p=p)
    torch.cuda.synchronize()
    assert_nan_parity(got.cpu().numpy(), ref, f"qsa token-id draft nan/{kernel}")


# ---------------------------------------------------------------------------
# every E4M3 code through the V decode (FP16) of both paths
# ---------------------------------------------------------------------------

def _v_probe_row() -> np.ndarray:
    """256 bytes: the 254 finite codes, then +0 and -0 again."""
    return np.concatenate([FINITE_CODES, np.array([0x00, 0x80], np.uint8)])


def _check_v_codes(out_rows: np.ndarray, what: str):
    """out_rows [n][256] float16 against fp16(decode(code)): bit for bit for
    nonzero codes, zero (either sign) for the two zero codes."""
    ref = torch.from_numpy(_v_probe_row()).view(torch.float8_e4m3fn).to(torch.float16).numpy()
    nz = ref != 0
    for r, row in enumerate(out_rows):
        assert np.array_equal(row[nz].view(np.uint16), ref[nz].view(np.uint16)), \
            f"{what}: row {r}, codes {_v_probe_row()[nz][row[nz] != ref[nz]][:8]}"
        assert not row[~nz].any(), f"{what}: zero codes, row {r}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_v_decode_every_code_dense(kernel):
    base = wl.make_dense("vcodes", 0xC0DE5, q_rows=2, num_heads=6, num_kv_heads=1,
                         head_dim=256, ctx=2048, page_size=800, pool_pages=6, sigma=1.0,
                         k_scale=1.0, v_scale=1.0, num_splits=4)
    probe = 1000
    lp, u = divmod(probe, base.page_size)
    phys = int(base.block_table[lp])
    k = np.zeros_like(base.k_pool)
    k[phys, u, 0, :] = 0x7E
    v = base.v_pool.copy()
    v[phys, u, 0, :] = _v_probe_row()
    ones = np.full(base.q_bits.shape, np.float16(1.0)).view(np.uint16)
    w = dataclasses.replace(base, k_pool=k, v_pool=v, q_bits=ones,
                            row_lens=np.array([2048, 2048], np.int32))
    announce("v codes dense", kernel)
    got = gu.run_dense(w, kernel)
    _check_v_codes(got.reshape(-1, 256), f"dense V decode/{kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_v_decode_every_code_sparse(kernel):
    base = wl.make_qsa("vcodes_qsa", 0xC0DE6, batch=1, q_rows=2, num_heads=6, num_kv_heads=1,
                       head_dim=256, ctx=2048, page_size=64, topk=8, k_scale=1.0,
                       v_scale=1.0, num_splits=2)
    newest = 2048 // 64 - 1
    blk = next(int(s) for s in base.sel_blocks[0, 0] if s != newest)
    phys, u = int(base.block_table[0, blk]), 5
    k = np.zeros_like(base.k_pool)
    k[phys, u, 0, :] = 0x7E
    v = base.v_pool.copy()
    v[phys, u, 0, :] = _v_probe_row()
    ones = np.full(base.q_bits.shape, 0x3F80, np.uint16)          # bf16 1.0
    w = dataclasses.replace(base, k_pool=k, v_pool=v, q_bits=ones)
    announce("v codes sparse", kernel)
    got = gu.run_qsa(w, kernel)
    _check_v_codes(got.reshape(-1, 256), f"sparse V decode/{kernel}")


# ---------------------------------------------------------------------------
# every E4M3 code through the K decode (FP16 dense, BF16 sparse)
# ---------------------------------------------------------------------------

def _expected_max(codes, sm_scale, k_scale) -> np.ndarray:
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    return dec * folded_scale(sm_scale, k_scale)


@pytest.mark.parametrize("kernel", KERNELS)
def test_k_decode_every_code_dense(kernel):
    n = FINITE_CODES.size
    base = wl.make_dense("kcodes", 0xC0DE7, q_rows=1, num_heads=6, num_kv_heads=1,
                         head_dim=256, ctx=64 * n, page_size=64, pool_pages=n + 2, sigma=1.0,
                         k_scale=0.75, v_scale=1.0, num_splits=n)
    k = base.k_pool.copy()
    for p in range(n):
        k[base.block_table[p]] = FINITE_CODES[p]
    q = np.zeros(base.q_bits.shape, np.uint16)
    q[..., 0] = 0x3C00                                              # fp16 1.0 on dim 0
    w = dataclasses.replace(base, k_pool=k, q_bits=q,
                            row_lens=np.array([64 * n], np.int32))
    announce("k codes dense", kernel)
    _, p, (acc, mx, sm) = gu.run_dense(w, kernel, return_ws=True)
    assert (p.num_splits, p.tokens_per_split) == (n, 64)
    exp = _expected_max(FINITE_CODES, w.sm_scale, w.k_scale)
    for r in range(mx.shape[1]):
        bad = np.nonzero(mx[:, r] != exp)[0]
        assert bad.size == 0, f"row {r}: codes {FINITE_CODES[bad][:8]} got {mx[bad[:4], r]}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_k_decode_every_code_sparse(kernel):
    n = FINITE_CODES.size
    base = wl.make_qsa("kcodes_qsa", 0xC0DE8, batch=1, q_rows=1, num_heads=2, num_kv_heads=1,
                       head_dim=256, ctx=64 * n, page_size=64, topk=n, k_scale=0.75,
                       v_scale=1.0, num_splits=n,
                       row_lens=np.array([[64 * n]], np.int32))
    k = base.k_pool.copy()
    for s in range(n):
        k[base.block_table[0, base.sel_blocks[0, 0, s]]] = FINITE_CODES[s]
    q = np.zeros(base.q_bits.shape, np.uint16)
    q[..., 0] = 0x3F80                                              # bf16 1.0 on dim 0
    w = dataclasses.replace(base, k_pool=k, q_bits=q)
    announce("k codes sparse", kernel)
    _, p, (acc, mx, sm) = gu.run_qsa(w, kernel, return_ws=True)
    assert (p.num_splits, p.tokens_per_split) == (n, 64)
    exp = _expected_max(FINITE_CODES, w.sm_scale, w.k_scale)
    for r in range(mx.shape[1]):
        bad = np.nonzero(mx[:, r] != exp)[0]
        assert bad.size == 0, f"row {r}: codes {FINITE_CODES[bad][:8]} got {mx[bad[:4], r]}"
