"""GPU parity: the HIP path through its C ABI against the FP64 oracle.

Every case prints a line naming itself before it touches the GPU.  Full-size
cases are the five named configurations in the split plan the benchmark
uses; small cases span several 64-token tiles with a ragged tail, odd page
sizes, grouped heads with more than one KV head, and forced split counts."""

import dataclasses

import numpy as np
import pytest
import torch

import fp8_kv_paged_attn_amd as pa
from fp8_kv_paged_attn_amd import workloads as wl
from tests import gpu_util as gu
from tests.oracle_pins import lse_merge

pytestmark = pytest.mark.gpu

KERNELS = ["simple", "mfma"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.require_gpu()
    pa.lib()


def announce(*what):
    print("[case]", *what, flush=True)


# ---------------------------------------------------------------------------
# the five named configurations
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("name", ["c0", "c1", "c2_16k", "c2_32k", "c2_64k", "c2_128k", "c3"])
def test_dense_config(orc, name, kernel):
    w = wl.cached(name)
    announce(name, kernel)
    got = gu.run_dense(w, kernel)
    ref = orc.dense_workload(w, nthreads=8)
    gu.assert_parity(got, ref, f"{name}/{kernel}")
    if name == "c3":
        assert not got[5:].any(), "zero-length rows must be exactly zero"


@pytest.mark.parametrize("kernel", KERNELS)
def test_qsa_config(orc, kernel):
    w = wl.cached("c4")
    announce("c4", kernel)
    got = gu.run_qsa(w, kernel)
    ref = orc.qsa_workload(w, nthreads=8)
    gu.assert_parity(got, ref, f"c4/{kernel}")


# ---------------------------------------------------------------------------
# small cases: tiles, ragged tails, page sizes, grouped heads, forced splits
# ---------------------------------------------------------------------------

SMALL = [
    # (q_rows, H, Hkv, D, ctx, page, lens, splits)
    (2, 6, 1, 256, 300, 48, None, 3),
    (8, 6, 1, 256, 1000, 800, None, 0),
    (3, 4, 2, 128, 517, 16, [0, 200, 517], 5),
    (1, 6, 1, 256, 70, 7, None, 1),
    (4, 12, 1, 128, 640, 64, [637, 638, 639, 640], 10),
    (8, 6, 1, 256, 2500, 848, [2493, 2494, 2495, 2496, 2497, 0, 0, 0], 0),
    (2, 24, 1, 256, 200, 16, None, 2),
    (5, 8, 4, 256, 333, 1, None, 4),
    (8, 6, 1, 256, 4100, 1728, None, 64),
    # a wave's next block 128 positions on in the same page (reference moved in
    # place) or past it (looked up): pages of 288 (wave 0's third block still
    # fits, the others cross), 1000 (not a multiple of 32: blocks straddle two
    # pages), 160 (only the first step of wave 0 stays) and 2048 with lengths
    # and a split end inside a page
    (8, 6, 1, 256, 3000, 288, None, 2),
    (4, 6, 1, 256, 2100, 1000, [2095, 2096, 2097, 2100], 3),
    (8, 6, 1, 256, 5000, 160, None, 4),
    (8, 6, 1, 256, 4000, 2048, [3990, 3991, 3992, 3993, 3994, 3995, 3996, 3997], 3),
]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_dense_small(orc, case, kernel):
    qr, H, Hkv, D, ctx, page, lens, splits = SMALL[case]
    npages = -(-ctx // page)
    w = wl.make_dense(f"small{case}", 0x5EED00 + case, q_rows=qr, num_heads=H, num_kv_heads=Hkv,
                      head_dim=D, ctx=ctx, page_size=page, pool_pages=npages + 3, sigma=1.2,
                      k_scale=0.45, v_scale=1.6, row_lens=lens, num_splits=splits,
                      poison_tail=True)
    announce("small", case, SMALL[case], kernel)
    got = gu.run_dense(w, kernel)
    ref = orc.dense_workload(w)
    gu.assert_parity(got, ref, f"small{case}/{kernel}")


# the MFMA kernel's row chunks: a unit's rows cut into workgroups of 16, 32 or
# 48 rows (ragged last chunks included) give the same function
CHUNKED = [
    # (q_rows, H, Hkv, D, ctx, page, lens, splits)
    (8, 6, 1, 256, 1000, 800, None, 3),                                    # 48 rows
    (7, 6, 1, 256, 2100, 1000, [2090, 2091, 2092, 2093, 2094, 2095, 2096], 2),   # 42
    (5, 4, 1, 128, 600, 64, [0, 100, 300, 599, 600], 4),                  # 20 rows
    (8, 6, 1, 256, 2500, 848, [2493, 2494, 2495, 2496, 2497, 0, 0, 0], 0),  # empty chunk
]


@pytest.mark.parametrize("chunk", [16, 32, 48])
@pytest.mark.parametrize("case", range(len(CHUNKED)))
def test_dense_row_chunks(orc, case, chunk):
    qr, H, Hkv, D, ctx, page, lens, splits = CHUNKED[case]
    w = wl.make_dense(f"chunk{case}", 0x5EED40 + case, q_rows=qr, num_heads=H, num_kv_heads=Hkv,
                      head_dim=D, ctx=ctx, page_size=page, pool_pages=-(-ctx // page) + 2,
                      sigma=1.2, k_scale=0.45, v_scale=1.6, row_lens=lens, num_splits=splits,
                      poison_tail=True)
    announce("row_chunks", case, CHUNKED[case], chunk)
    got = gu.run_dense(w, "mfma", rows_per_workgroup=chunk)
    gu.assert_parity(got, orc.dense_workload(w), f"chunk{case}/{chunk}")


@pytest.mark.parametrize("chunk", [16, 32])
def test_qsa_row_chunks(orc, chunk):
    w = wl.make_qsa("qsa_chunk", 0x5EED51, batch=3, q_rows=4, num_heads=12, num_kv_heads=2,
                    head_dim=128, ctx=1024, page_size=64, topk=6, k_scale=0.5, v_scale=2.0,
                    num_splits=3)
    announce("qsa_row_chunks", chunk)
    got = gu.run_qsa(w, "mfma", rows_per_workgroup=chunk)
    gu.assert_parity(got, orc.qsa_workload(w), f"qsa_chunk/{chunk}")


def test_plan_picks_row_chunks_c1():
    """The full-size 8K workload runs with 16-row chunks (its parity test above
    goes through this plan)."""
    w = wl.cached("c1")
    assert gu.dense_plan(w, "auto", None).rows_per_workgroup == 16


@pytest.mark.parametrize("kernel", KERNELS)
def test_qsa_small_edges(orc, kernel):
    w = wl.make_qsa("qsa_small", 0x5EED50, batch=3, q_rows=4, num_heads=12, num_kv_heads=2,
                    head_dim=128, ctx=1024, page_size=64, topk=6, k_scale=0.5, v_scale=2.0,
                    num_splits=3)
    sel = w.sel_blocks.copy()
    sel[0, 0, 2] = -1                       # empty slot
    sel[1, 1, 0] = sel[1, 1, 3]             # a block listed twice
    sel[2, 0, :] = -1                       # nothing selected
    lens = w.row_lens.copy()
    lens[0, 1] = 0
    lens[1, :] = [1000, 1001, 1002, 5000]   # the last is clamped to 1024
    w = dataclasses.replace(w, sel_blocks=sel, row_lens=lens)
    announce("qsa_small_edges", kernel)
    got = gu.run_qsa(w, kernel)
    ref = orc.qsa_workload(w)
    gu.assert_parity(got, ref, f"qsa_small/{kernel}")
    assert not got[2, :, :6].any(), "unit with an empty selection must give zeros"
    assert not got[0, 1].any()


@pytest.mark.parametrize("kernel", KERNELS)
def test_qsa_d256(orc, kernel):
    w = wl.make_qsa("qsa_d256", 0x5EED51, batch=2, q_rows=8, num_heads=6, num_kv_heads=1,
                    head_dim=256, ctx=640, page_size=32, topk=5, k_scale=0.37, v_scale=1.9)
    announce("qsa_d256", kernel)
    gu.assert_parity(gu.run_qsa(w, kernel), orc.qsa_workload(w), f"qsa_d256/{kernel}")


# ---------------------------------------------------------------------------
# sparse verify over selected token ids
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_qsa_tokens_config(orc, kernel):
    w = wl.cached("c4tok")
    announce("c4tok", kernel)
    got = gu.run_qsa_tokens(w, kernel)
    gu.assert_parity(got, orc.qsa_tokens_workload(w, nthreads=8), f"c4tok/{kernel}")


def _tokens_edges(seed, **kw):
    w = wl.make_qsa_tokens(f"tok_edges{seed}", seed, **kw)
    sel = w.sel_tokens.copy()
    cap = w.max_blocks * w.page_size
    sel[0, 0, 5] = sel[0, 0, 9]             # an id listed twice
    sel[0, -1, 3] = cap + 5                 # an id past the table: never seen
    sel[-1, 0, :] = -1                      # nothing selected
    lens = w.row_lens.copy()
    lens[0, 1] = 0
    lens[1, -1] = 10 ** 6                   # clamped to the table's capacity
    return dataclasses.replace(w, sel_tokens=sel, row_lens=lens)


TOKEN_EDGES = [
    # (D, heads, kv heads, q rows, ctx, page, ids per list, -1 entries, splits)
    (128, 12, 2, 4, 1500, 64, 300, 7, 3),
    (128, 24, 2, 4, 2000, 16, 700, 0, None),
    (256, 6, 1, 8, 900, 32, 250, 5, 2),
    (256, 6, 1, 3, 700, 7, 129, 1, 1),
]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", range(len(TOKEN_EDGES)))
def test_qsa_tokens_small_edges(orc, case, kernel):
    D, H, Hkv, qr, ctx, ps, n, empty, splits = TOKEN_EDGES[case]
    w = _tokens_edges(0x70C0 + case, batch=3, q_rows=qr, num_heads=H, num_kv_heads=Hkv,
                      head_dim=D, ctx=ctx, page_size=ps, num_sel=n, num_empty=empty,
                      k_scale=0.5, v_scale=2.0, num_splits=splits or 0)
    announce("qsa_tokens_edges", TOKEN_EDGES[case], kernel)
    got = gu.run_qsa_tokens(w, kernel)
    gu.assert_parity(got, orc.qsa_tokens_workload(w), f"tokens{case}/{kernel}")
    G = H // Hkv
    assert not got[2, :, :G].any(), "unit with an empty selection must give zeros"
    assert not got[0, 1].any(), "zero-length row"


@pytest.mark.parametrize("kernel", KERNELS)
def test_qsa_tokens_match_block_selection(kernel):
    """A block selection written out as token ids gives the block entry's
    output bit for bit: same tokens, same list order, same splits."""
    qb = wl.make_qsa("tok_vs_blk", 0x70D0, batch=2, q_rows=4, num_heads=12, num_kv_heads=2,
                     head_dim=128, ctx=2048, page_size=64, topk=6, k_scale=0.5, v_scale=2.0,
                     num_splits=3)
    sel = qb.sel_blocks.copy()
    sel[1, 0, 2] = -1
    qb = dataclasses.replace(qb, sel_blocks=sel)
    tok = wl.tokens_from_blocks(qb)
    qt = wl.QsaTokensWorkload(
        name="tok_vs_blk_t", q_bits=qb.q_bits, k_pool=qb.k_pool, v_pool=qb.v_pool,
        block_table=qb.block_table, sel_tokens=tok, row_lens=qb.row_lens, batch=qb.batch,
        q_rows=qb.q_rows, num_heads=qb.num_heads, num_kv_heads=qb.num_kv_heads,
        head_dim=qb.head_dim, page_size=qb.page_size, max_blocks=qb.max_blocks,
        num_sel=tok.shape[2], sm_scale=qb.sm_scale, k_scale=qb.k_scale, v_scale=qb.v_scale,
        num_splits=3)
    announce("tokens_vs_blocks", kernel)
    a = gu.run_qsa(qb, kernel)
    b = gu.run_qsa_tokens(qt, kernel)
    assert np.all(np.isfinite(b)), "token ids reached a poisoned page"
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("kernel", KERNELS)
def test_qsa_tokens_unseen_bytes_never_read(kernel):
    """NaN bytes at every token no row of its (request, KV head) sees (not
    selected, or selected at or past the longest row) change no output bit."""
    w = _tokens_edges(0x70E0, batch=3, q_rows=4, num_heads=12, num_kv_heads=2, head_dim=128,
                      ctx=1500, page_size=64, num_sel=300, num_empty=7, k_scale=0.5,
                      v_scale=2.0, num_splits=3)
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    seen = np.zeros(kp.shape[:3], bool)
    cap = w.max_blocks * w.page_size
    for b in range(w.batch):
        lmax = min(max(int(w.row_lens[b].max()), 0), cap)
        for g in range(w.num_kv_heads):
            for t in w.sel_tokens[b, g]:
                if 0 <= t < lmax:
                    seen[w.block_table[b, t // w.page_size], t % w.page_size, g] = True
    kp[~seen] = 0x7F
    vp[~seen] = 0xFF
    announce("tokens_unseen_nan", kernel)
    clean = gu.run_qsa_tokens(w, kernel)
    dirty = gu.run_qsa_tokens(w, kernel, k_pool=kp, v_pool=vp)
    assert np.array_equal(clean.view(np.uint16), dirty.view(np.uint16))


def test_qsa_tokens_long_split_kernel_choice(orc):
    """A list longer than the MFMA kernel's slot cache asked for in one split:
    the planner raises the split count so that the MFMA kernel takes it (auto
    and mfma match the oracle); a hand-made one-split plan is refused by the
    MFMA kernel and runs only on the plain kernel, when asked for."""
    w = wl.make_qsa_tokens("tok_long", 0x70F0, batch=1, q_rows=2, num_heads=6, num_kv_heads=1,
                           head_dim=256, ctx=3000, page_size=64, num_sel=1100, num_empty=4,
                           k_scale=0.5, v_scale=2.0, num_splits=1)
    announce("tokens_long_split")
    ref = orc.qsa_tokens_workload(w)
    for kernel in ("auto", "mfma"):
        gu.assert_parity(gu.run_qsa_tokens(w, kernel), ref, f"tok_long {kernel}")
    q = gu.bf16_tensor(w.q_bits).to(gu.DEV)
    k = torch.from_numpy(w.k_pool).to(gu.DEV)
    v = torch.from_numpy(w.v_pool).to(gu.DEV)
    bt = torch.from_numpy(w.block_table.astype(np.int32)).to(gu.DEV)
    sel = torch.from_numpy(w.sel_tokens.astype(np.int32)).to(gu.DEV)
    lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(gu.DEV)
    p = pa.plan(w.num_sel, w.q_rows * w.num_heads, 1, w.head_dim, w.page_size, "tokens",
                splits=1)
    assert p.num_splits == 2
    p.num_splits, p.tokens_per_split = 1, 1152
    p.ws_acc_bytes, p.ws_stat_bytes = p.ws_acc_bytes // 2, p.ws_stat_bytes // 2
    run = lambda: pa.qsa_verify_tokens(q, k, v, bt, sel, lens, sm_scale=w.sm_scale,
                                       k_scale=w.k_scale, v_scale=w.v_scale, p=p)
    for kernel in ("auto", "mfma"):
        p.kernel = pa.PA_KERNEL[kernel]
        with pytest.raises(RuntimeError, match="-7|plan"):
            run()
    p.kernel = pa.PA_KERNEL["simple"]
    got = run()
    torch.cuda.synchronize()
    gu.assert_parity(got.cpu().numpy(), ref, "tok_long simple, one split")


# ---------------------------------------------------------------------------
# workspace and combine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_workspace_partials_c0(orc, kernel):
    """The FP32 split workspace is part of the interface: compare it with the
    oracle's split partials, and the combine kernel with the oracle's combine
    of the same FP32 workspace (within one FP16 ulp)."""
    w = wl.cached("c0")
    announce("workspace c0", kernel)
    got, p, (acc, mx, sm) = gu.run_dense(w, kernel, return_ws=True)
    assert p.num_splits == 4
    oacc, omx, osm = orc.verify_dense_split(w.q_bits, w.k_pool, w.v_pool, w.block_table,
                                            w.row_lens, w.max_tokens, w.num_kv_heads,
                                            w.sm_scale, w.k_scale, p.num_splits,
                                            p.tokens_per_split)
    assert np.allclose(mx, omx, rtol=2e-6, atol=2e-5), np.abs(mx - omx).max()
    assert np.allclose(sm, osm, rtol=2e-5, atol=0), np.abs(sm / osm - 1).max()
    nz = osm > 0
    norm_gpu = acc[nz] / sm[nz][:, None]
    norm_orc = oacc[nz] / osm[nz][:, None]
    rel = np.linalg.norm(norm_gpu - norm_orc) / np.linalg.norm(norm_orc)
    assert rel < 1e-4, rel
    comb = orc.combine(acc, mx, sm, w.v_scale).reshape(got.shape)
    ulp = np.spacing(np.abs(comb).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - comb) <= ulp), "combine off by > 1 fp16 ulp"


@pytest.mark.parametrize("kernel", KERNELS)
def test_empty_split_numerators_unused(orc, kernel):
    """An empty split's numerator (sum 0) need not be written and is never
    used: with the workspace filled with NaN before the call, rows of length
    zero still come out exactly zero, every other row meets the parity bar,
    and every split with a nonzero sum has its numerator written (finite)."""
    w = wl.make_dense("empty_num", 0xE3B7, q_rows=6, num_heads=6, num_kv_heads=1,
                      head_dim=256, ctx=1500, page_size=160, pool_pages=12, sigma=1.0,
                      k_scale=0.5, v_scale=1.5, row_lens=[1495, 0, 700, 0, 0, 1500],
                      num_splits=6)
    announce("empty split numerators", kernel)
    d = gu.dense_to_dev(w)
    p = gu.dense_plan(w, kernel)
    ws = pa.make_workspace(p, w.q_rows * w.num_heads, w.head_dim, gu.DEV)
    for t in ws:
        t.fill_(float("nan"))
    out = pa.verify(d.q, d.k, d.v, d.table, d.lens, w.max_tokens, sm_scale=w.sm_scale,
                    k_scale=w.k_scale, v_scale=w.v_scale, p=p, ws=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    acc, mx, sm = (t.cpu().numpy() for t in ws)
    assert not np.isnan(mx).any() and not np.isnan(sm).any()
    assert np.isfinite(acc[sm != 0]).all()
    assert (sm == 0).any(), "the case must have empty splits"
    assert not got[[1, 3, 4]].any(), "zero-length rows must be exactly zero"
    gu.assert_parity(got, orc.dense_workload(w), f"empty split numerators/{kernel}")


def test_combine_empty_and_single_split():
    """Combine edge cases fed directly: every split empty -> 0; one split ->
    out_scale * acc / sum."""
    S, R, D = 3, 5, 256
    acc = torch.zeros((S, R, D), dtype=torch.float32, device=gu.DEV)
    mx = torch.full((S, R), float("-inf"), device=gu.DEV)
    sm = torch.zeros((S, R), device=gu.DEV)
    acc[1, 2] = torch.arange(D, dtype=torch.float32, device=gu.DEV)
    mx[1, 2] = 3.0
    sm[1, 2] = 2.0
    out = torch.full((R, D), 7.0, dtype=torch.float16, device=gu.DEV)
    announce("combine edges")
    pa.paged_attn_combine_fp32((acc, mx, sm), S, R, D, 1.5, out)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    exp = np.zeros((R, D))
    exp[2] = (np.arange(D) / 2.0 * 1.5).astype(np.float16)
    assert np.array_equal(o, exp)


def _random_partials(S, R, D, seed):
    """FP32 split partials with maxima spread over many binades and about a
    third of the (split, row) pairs empty (m = -inf, l = 0, acc = 0); row 3 is
    empty in every split."""
    rng = np.random.default_rng(seed)
    mx = rng.normal(0.0, 8.0, (S, R)).astype(np.float32)
    sm = rng.uniform(0.5, 40.0, (S, R)).astype(np.float32)
    acc = (rng.normal(0.0, 1.0, (S, R, D)) * sm[..., None]).astype(np.float32)
    empty = rng.random((S, R)) < 0.3
    empty[:, 3] = True
    mx[empty] = -np.inf
    sm[empty] = 0.0
    acc[empty] = 0.0
    return acc, mx, sm, empty


def _combine(acc, mx, sm, v_scale, lse=False):
    S, R, D = acc.shape
    dev = [torch.from_numpy(np.ascontiguousarray(x)).to(gu.DEV) for x in (acc, mx, sm)]
    out = torch.empty((R, D), dtype=torch.float16, device=gu.DEV)
    if not lse:
        pa.paged_attn_combine_fp32(tuple(dev), S, R, D, v_scale, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()
    o32 = torch.empty(R * D, dtype=torch.float32, device=gu.DEV)
    l32 = torch.empty(R, dtype=torch.float32, device=gu.DEV)
    pa.paged_attn_combine_fp32_lse(tuple(dev), S, R, D, v_scale, out=out, out32=o32, lse=l32)
    torch.cuda.synchronize()
    return out.cpu().numpy(), o32.cpu().numpy().reshape(R, D), l32.cpu().numpy()


@pytest.mark.parametrize("S", [37, 300, 700])
def test_combine_many_splits(orc, S):
    """More splits than one batch per thread (12 rows get 16 split groups, so
    300 and 700 splits take 2 and 3 batches of 16, 37 one partial batch): the
    running state is rescaled from batch to batch.  The FP16 output is within
    1 fp16 ulp of the oracle's FP64 merge of the same FP32 partials, the FP32
    output and LSE within FP32 rounding, and a row with every split empty gives
    zeros and LSE -inf.  Garbage (NaN, inf) in the accumulators of empty splits
    changes no output bit: an empty split's numerator is never used."""
    R, D, v_scale = 12, 256, 1.7
    announce("combine many splits", S)
    acc, mx, sm, empty = _random_partials(S, R, D, 0xC0B1 + S)
    ref, ref_lse = orc.combine(acc, mx, sm, v_scale, with_lse=True)
    got16, got32, gl = _combine(acc, mx, sm, v_scale, lse=True)
    ulp = np.spacing(np.abs(ref).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got16.astype(np.float64) - ref) <= ulp), "combine off by > 1 fp16 ulp"
    assert np.abs(got32 - ref).max() <= 2e-6 * np.abs(ref).max()
    live = np.isfinite(ref_lse)
    assert not live[3] and gl[3] == -np.inf and not got16[3].any() and not got32[3].any()
    assert np.all(np.abs(gl[live] - ref_lse[live]) <= 2e-6 * np.maximum(1.0, np.abs(ref_lse[live])))
    dirty = acc.copy()
    dirty[empty] = np.nan
    dirty[empty & (np.arange(S)[:, None] % 2 == 0)] = np.inf
    assert np.array_equal(_combine(dirty, mx, sm, v_scale).view(np.uint16),
                          got16.view(np.uint16)), "empty-split accumulators leaked"


def test_combine_nan_sum_reaches_row():
    """A split whose sum is NaN is not empty: its row becomes NaN, also when
    its max is -inf (every score it saw was NaN) and when it is the row's only
    non-empty split; the other rows are unaffected."""
    S, R, D = 300, 12, 256
    announce("combine NaN sums")
    acc, mx, sm, empty = _random_partials(S, R, D, 0xC0B2)
    clean = _combine(acc, mx, sm, 1.0)
    sm2, mx2 = sm.copy(), mx.copy()
    sm2[7, 5] = np.nan                       # row 5: NaN sum, finite max
    sm2[:, 6] = 0.0                          # row 6: only split 250, NaN sum, max -inf
    mx2[:, 6] = -np.inf
    sm2[250, 6] = np.nan
    sm2[40, 8], mx2[40, 8] = np.nan, -np.inf  # row 8: NaN sum, max -inf, among live splits
    got = _combine(acc, mx2, sm2, 1.0)
    for r in (5, 6, 8):
        assert np.isnan(got[r].astype(np.float32)).all(), f"row {r} must be NaN"
    keep = [r for r in range(R) if r not in (5, 6, 8)]
    assert np.array_equal(got[keep].view(np.uint16), clean[keep].view(np.uint16))


# ---------------------------------------------------------------------------
# index handling: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_one_hot_probe_bit_exact(orc, kernel):
    """K = 448 on one token, zero elsewhere, q = 1: the softmax is one-hot in
    FP32 too, so every row returns fp16(v_scale * V[probe]) exactly, for probes
    at page starts and ends, in the partial last page and past a split edge."""
    base = wl.make_dense("probe", 0x9B0BE, q_rows=2, num_heads=6, num_kv_heads=1, head_dim=256,
                         ctx=2048, page_size=800, pool_pages=6, sigma=1.0, k_scale=1.0,
                         v_scale=1.5, num_splits=4)
    ones = np.full(base.q_bits.shape, np.float16(1.0)).view(np.uint16)
    tab = orc.e4m3_table()
    for probe in [0, 511, 512, 799, 800, 1599, 1600, 2046, 2047]:
        k = np.zeros_like(base.k_pool)
        lp, u = divmod(probe, base.page_size)
        phys = int(base.block_table[lp])
        k[phys, u, 0, :] = 0x7E
        w = dataclasses.replace(base, k_pool=k, q_bits=ones,
                                row_lens=np.array([2048, 2048], np.int32))
        announce("probe", probe, kernel)
        got = gu.run_dense(w, kernel)
        exp = (np.float32(w.v_scale) * tab[base.v_pool[phys, u, 0]].astype(np.float32)
               ).astype(np.float16)
        assert np.array_equal(got[0, 0], exp) and np.array_equal(got[1, 5], exp), probe


@pytest.mark.parametrize("kernel", KERNELS)
def test_relocation_and_strided_view_bit_identical(kernel):
    """Pages moved to other physical slots, and the pool read as a strided view
    of a packed allocation (two members interleaved per page), give
    bit-identical output under the same plan."""
    w = wl.make_dense("reloc", 0x7E10C, q_rows=8, num_heads=6, num_kv_heads=1, head_dim=256,
                      ctx=3000, page_size=848, pool_pages=8, sigma=1.5, k_scale=0.37,
                      v_scale=1.9)
    announce("relocation", kernel)
    base = gu.run_dense(w, kernel)
    P = w.k_pool.shape[0]
    perm = np.roll(np.arange(P), 3)
    k = np.empty_like(w.k_pool)
    v = np.empty_like(w.v_pool)
    k[perm] = w.k_pool
    v[perm] = w.v_pool
    w2 = dataclasses.replace(w, k_pool=k, v_pool=v,
                             block_table=perm[w.block_table].astype(np.int32))
    assert np.array_equal(gu.run_dense(w2, kernel), base), "relocated pages"
    # packed: [P][page][2 members][Hkv][D]; this pool is member 1
    packed_k = torch.zeros((P, w.page_size, 2, 1, 256), dtype=torch.uint8, device=gu.DEV)
    packed_v = torch.full((P, w.page_size, 2, 1, 256), 0x7F, dtype=torch.uint8, device=gu.DEV)
    packed_k[:, :, 1] = torch.from_numpy(w.k_pool).to(gu.DEV)
    packed_v[:, :, 1] = torch.from_numpy(w.v_pool).to(gu.DEV)
    kview, vview = packed_k[:, :, 1], packed_v[:, :, 1]
    assert kview.stride(1) == 512
    got = gu.run_dense(w, kernel, k=kview, v=vview)
    assert np.array_equal(got, base), "strided view"


@pytest.mark.parametrize("kernel", KERNELS)
def test_nan_poison_bit_identical(kernel):
    """NaN bytes in the null page that pads the table, in page tails past the
    longest row and in unused pages leave the output bit-identical."""
    kw = dict(q_rows=8, num_heads=6, num_kv_heads=1, head_dim=256, ctx=3000, page_size=848,
              pool_pages=6, sigma=1.0, k_scale=0.5, v_scale=2.25,
              row_lens=[2996, 2997, 2998, 2999, 3000, 0, 0, 0], pad_table_to=8)
    clean = wl.make_dense("clean", 0x4A4, null_page_nan=True, poison_tail=False,
                          poison_unused=False, **kw)
    dirty = wl.make_dense("dirty", 0x4A4, null_page_nan=True, poison_tail=True,
                          poison_unused=True, **kw)
    clean = dataclasses.replace(clean, k_pool=clean.k_pool.copy(), v_pool=clean.v_pool.copy())
    clean.k_pool[0] = 0
    clean.v_pool[0] = 0
    assert (dirty.k_pool[0] == 0x7F).all()
    announce("nan poison", kernel)
    a = gu.run_dense(clean, kernel)
    b = gu.run_dense(dirty, kernel)
    assert np.all(np.isfinite(b.astype(np.float64)))
    assert np.array_equal(a, b)
    assert not b[5:].any()


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("splits", [0, 1])
def test_visible_nan_propagates(orc, kernel, splits):
    """NaN bytes at positions a row sees reach the output as in the oracle: a
    NaN K byte makes the rows seeing that token NaN, a NaN V byte makes one
    column NaN; everything else matches the oracle at the usual bar, with one
    split and with the planner's splits."""
    w = wl.make_dense("vnan", 0x7A7, q_rows=4, num_heads=6, num_kv_heads=1, head_dim=256,
                      ctx=700, page_size=96, pool_pages=9, sigma=1.0, k_scale=0.5,
                      v_scale=1.5, row_lens=[700, 640, 120, 0], num_splits=splits)
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    tk, tv, dv = 660, 100, 7              # token 660: row 0 only; token 100: rows 0-2
    k[w.block_table[tk // w.page_size], tk % w.page_size, 0, 11] = 0x7F
    v[w.block_table[tv // w.page_size], tv % w.page_size, 0, dv] = 0xFF
    w = dataclasses.replace(w, k_pool=k, v_pool=v)
    announce("visible nan", kernel, splits)
    got = gu.run_dense(w, kernel).astype(np.float64)
    ref = orc.dense_workload(w)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(ref[0]).all() and np.isnan(ref[1:3, :, dv]).all() and not ref[3].any()
    fin = np.isfinite(ref)
    gu.assert_parity(got[fin], ref[fin], f"visible nan/{kernel}/S{splits}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_zero_lengths(kernel):
    w = wl.make_dense("zeros", 0x2E0, q_rows=4, num_heads=6, num_kv_heads=1, head_dim=256,
                      ctx=700, page_size=96, pool_pages=9, sigma=1.0, k_scale=1.0, v_scale=1.0,
                      row_lens=[0, 0, 0, 0])
    announce("all rows empty", kernel)
    assert not gu.run_dense(w, kernel).any()
    w0 = dataclasses.replace(w, max_tokens=0)
    announce("max_tokens 0", kernel)
    assert not gu.run_dense(w0, kernel).any()


@pytest.mark.parametrize("kernel", KERNELS)
def test_length_clamp(orc, kernel):
    w = wl.make_dense("clamp", 0xC1A, q_rows=3, num_heads=6, num_kv_heads=1, head_dim=256,
                      ctx=500, page_size=64, pool_pages=10, sigma=1.0, k_scale=0.8,
                      v_scale=1.1, row_lens=[-5, 10**6, 250])
    announce("clamp", kernel)
    got = gu.run_dense(w, kernel)
    gu.assert_parity(got, orc.dense_workload(w), f"clamp/{kernel}")
    assert not got[0].any()


# ---------------------------------------------------------------------------
# graph replay with changed lengths
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_graph_replay_changed_lengths(kernel):
    """verify + combine captured once, replayed with new device lengths
    (including zeros) between eager work: each replay equals the eager call."""
    w = wl.make_dense("graph", 0x62A9, q_rows=8, num_heads=6, num_kv_heads=1, head_dim=256,
                      ctx=5000, page_size=1648, pool_pages=6, sigma=1.0, k_scale=0.6,
                      v_scale=1.3)
    d = gu.dense_to_dev(w)
    p = gu.dense_plan(w, kernel)
    ws = pa.make_workspace(p, 48, 256, gu.DEV)
    out = torch.empty((8, 6, 256), dtype=torch.float16, device=gu.DEV)
    lens = d.lens.clone()

    def step():
        pa.verify(d.q, d.k, d.v, d.table, lens, w.max_tokens, sm_scale=w.sm_scale,
                  k_scale=w.k_scale, v_scale=w.v_scale, p=p, ws=ws, out=out)

    announce("graph capture", kernel)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    trials = [[4993, 4994, 4995, 4996, 4997, 4998, 4999, 5000], [0] * 8,
              [100, 0, 3000, 0, 5000, 1, 64, 65], [4993, 4994, 4995, 4996, 4997, 0, 0, 0]]
    for lv in trials:
        lens.copy_(torch.tensor(lv, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        replayed = out.cpu().numpy().copy()
        out.fill_(0)
        step()                              # eager, same buffers
        torch.cuda.synchronize()
        eager = out.cpu().numpy().copy()
        assert np.array_equal(replayed, eager), lv
        zero_rows = [i for i, x in enumerate(lv) if x == 0]
        assert not replayed[zero_rows].any()


def _capture(fn):
    """fn captured into a HIP graph after one eager run on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_match_eager(fn, outs, mutate):
    """Replay the captured fn after each input change, then run fn eagerly on
    the same buffers: every replay equals the eager result bit for bit."""
    g = _capture(fn)
    for k in range(3):
        mutate(k)
        for o in outs:                      # what a call leaves untouched stays zero
            o.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        replayed = [o.cpu().clone() for o in outs]
        for o in outs:
            o.fill_(0)
        fn()
        torch.cuda.synchronize()
        for r, o in zip(replayed, outs):
            assert torch.equal(r.view(torch.uint8), o.cpu().view(torch.uint8)), k


def test_graph_replay_sparse_and_batch_entries():
    """Each remaining verify entry, with its combine, is graph-capturable (no
    host synchronisation, no allocation) and replays with new device lengths."""
    qb = wl.make_qsa("graph_qsa", 0x62B0, batch=2, q_rows=4, num_heads=12, num_kv_heads=2,
                     head_dim=128, ctx=1024, page_size=64, topk=5, k_scale=0.5, v_scale=2.0,
                     num_splits=3)
    qt = wl.make_qsa_tokens("graph_tok", 0x62B1, batch=2, q_rows=4, num_heads=12,
                            num_kv_heads=2, head_dim=128, ctx=1024, page_size=64, num_sel=300,
                            num_empty=4, k_scale=0.5, v_scale=2.0, num_splits=3)
    wb = BATCHES_GRAPH()
    announce("graph capture: qsa blocks, qsa tokens, batch")
    dev = gu.DEV
    for kind, w in (("blocks", qb), ("tokens", qt), ("batch", wb)):
        if kind == "batch":
            q = gu.fp16_tensor(w.q_bits).to(dev)
        else:
            q = gu.bf16_tensor(w.q_bits).to(dev)
        k = torch.from_numpy(w.k_pool).to(dev)
        v = torch.from_numpy(w.v_pool).to(dev)
        bt = torch.from_numpy(w.block_table.astype(np.int32)).to(dev)
        lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(dev)
        B, qr, H, D = w.q_bits.shape
        out = torch.empty((B, qr, H, D), dtype=torch.float16, device=dev)
        G = H // w.num_kv_heads
        if kind == "blocks":
            sel = torch.from_numpy(w.sel_blocks.astype(np.int32)).to(dev)
            p = pa.plan(w.topk * w.page_size, qr * G, B * w.num_kv_heads, D, w.page_size,
                        "blocks", splits=3)
            fn = lambda: pa.qsa_verify(q, k, v, bt, sel, lens, sm_scale=w.sm_scale,
                                       k_scale=w.k_scale, v_scale=w.v_scale, p=p, ws=ws, out=out)
        elif kind == "tokens":
            sel = torch.from_numpy(w.sel_tokens.astype(np.int32)).to(dev)
            p = pa.plan(w.num_sel, qr * G, B * w.num_kv_heads, D, w.page_size, "tokens",
                        splits=3)
            fn = lambda: pa.qsa_verify_tokens(q, k, v, bt, sel, lens, sm_scale=w.sm_scale,
                                              k_scale=w.k_scale, v_scale=w.v_scale, p=p, ws=ws,
                                              out=out)
        else:
            p = pa.plan(w.cap, qr * G, B * w.num_kv_heads, D, w.page_size, "batch", splits=4)
            fn = lambda: pa.verify_batch(q, k, v, bt, lens, sm_scale=w.sm_scale,
                                         k_scale=w.k_scale, v_scale=w.v_scale, p=p, ws=ws,
                                         out=out)
        ws = pa.make_workspace(p, B * qr * H, D, dev)
        base = w.row_lens.astype(np.int64)
        trials = [base, np.zeros_like(base), np.maximum(base - 700, 0)]

        def mutate(i, lens=lens, trials=trials):
            lens.copy_(torch.from_numpy(trials[i].astype(np.int32)))

        _replays_match_eager(fn, [out], mutate)


def BATCHES_GRAPH():
    return wl.make_dense_batch("graph_batch", 0x62B2, q_rows=12, num_heads=6, num_kv_heads=1,
                               head_dim=256, ctxs=[900, 2500, 1700], page_size=256,
                               sigma=1.0, k_scale=0.5, v_scale=2.0)


def test_graph_replay_combine_lse_and_cache_write():
    """The LSE combine and the cache writer replay from a graph bit for bit."""
    announce("graph capture: combine with LSE, cache write")
    dev = gu.DEV
    S, R, D = 7, 40, 128
    gen = torch.Generator().manual_seed(0x62B3)
    acc = torch.randn((S, R, D), generator=gen).to(dev)
    mx = torch.randn((S, R), generator=gen).to(dev)
    sm = torch.rand((S, R), generator=gen).to(dev)
    out16 = torch.empty((R, D), dtype=torch.float16, device=dev)
    out32 = torch.empty((R, D), dtype=torch.float32, device=dev)
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    fn = lambda: pa.paged_attn_combine_fp32_lse((acc, mx, sm), S, R, D, 1.7, out=out16,
                                                out32=out32, lse=lse)

    def mutate(i):
        sm[:, i * 5:(i + 1) * 5] = 0.0          # some rows lose splits, one row all of them
        sm[:, 39] = 0.0

    _replays_match_eager(fn, [out16, out32, lse], mutate)

    T, Hkv, Dh, page = 300, 2, 64, 16
    kx = torch.randn((T, Hkv, Dh), generator=gen).to(torch.float16).to(dev)
    vx = torch.randn((T, Hkv, Dh), generator=gen).to(torch.float16).to(dev)
    slots = torch.randperm(40 * page, generator=gen)[:T].to(torch.int64).to(dev)
    kp = torch.zeros((40, page, Hkv, Dh), dtype=torch.uint8, device=dev)
    vp = torch.zeros_like(kp)
    fn2 = lambda: pa.paged_attn_cache_write_e4m3(kx, vx, slots, kp, vp, 0.37, 2.25)

    def mutate2(i):
        kx.mul_(-1.5)
        slots[i::7] = -1                        # skipped tokens

    _replays_match_eager(fn2, [kp, vp], mutate2)


# ---------------------------------------------------------------------------
# kernel timer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kernel", KERNELS)
def test_kernel_timer(kernel):
    """Timed launches give the same bytes as untimed ones; the timer records
    exactly the armed number of launches, each inside the bracketing events."""
    w = wl.make_dense("timer", 0x7133, q_rows=8, num_heads=6, num_kv_heads=1, head_dim=256,
                      ctx=9000, page_size=1648, pool_pages=8, sigma=1.0, k_scale=0.7,
                      v_scale=1.2)
    d = gu.dense_to_dev(w)
    announce("timer untimed", kernel)
    ref = gu.run_dense(w, kernel, d=d)
    announce("timer armed", kernel)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    pa.timer_arm(2)
    t0.record()
    outs = [gu.run_dense(w, kernel, d=d) for _ in range(3)]
    t1.record()
    torch.cuda.synchronize()
    ms = pa.timer_read()
    assert len(ms) == 2
    total = t0.elapsed_time(t1)
    assert all(0.0 < x < total for x in ms), (ms, total)
    for o in outs:
        assert np.array_equal(o, ref)
    assert pa.timer_read() == []            # reading disarmed it


def test_stream_read_probe_runs():
    """The read probe reads a zero buffer without touching its sink."""
    announce("stream read probe")
    buf = torch.zeros(1 << 20, 4, dtype=torch.int32, device=gu.DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=gu.DEV)
    pa.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


# ---------------------------------------------------------------------------
# combine with the base-2 LSE (merge across ranks)
# ---------------------------------------------------------------------------

def _c3_workspace():
    w = wl.cached("c3")
    d = gu.dense_to_dev(w)
    p = gu.dense_plan(w, "mfma")
    ws = pa.make_workspace(p, w.q_rows * w.num_heads, w.head_dim, gu.DEV)
    pa.paged_attn_verify_e4m3(d.q, d.k, d.v, d.table, d.lens, w.max_tokens, w.sm_scale,
                              w.k_scale, p, ws)
    return w, p, ws


def test_combine_lse_matches_oracle(orc):
    """The LSE combine's FP16 output is bit-identical to the plain combine's; its
    FP32 output and LSE match the FP64 oracle merge of the same FP32 partials
    (FP32 rounding only); empty rows give LSE -inf and zeros."""
    announce("combine lse c3")
    w, p, ws = _c3_workspace()
    R, D = w.q_rows * w.num_heads, w.head_dim
    out16 = torch.empty(R * D, dtype=torch.float16, device=gu.DEV)
    ref16 = torch.empty(R * D, dtype=torch.float16, device=gu.DEV)
    out32 = torch.empty(R * D, dtype=torch.float32, device=gu.DEV)
    lse = torch.empty(R, dtype=torch.float32, device=gu.DEV)
    pa.paged_attn_combine_fp32(ws, p.num_splits, R, D, w.v_scale, ref16)
    pa.paged_attn_combine_fp32_lse(ws, p.num_splits, R, D, w.v_scale, out=out16, out32=out32,
                                   lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out16, ref16)
    S = p.num_splits
    acc = ws[0].cpu().numpy().reshape(S, R, D)
    mx = ws[1].cpu().numpy().reshape(S, R)
    sm = ws[2].cpu().numpy().reshape(S, R)
    ref_out, ref_lse = orc.combine(acc, mx, sm, w.v_scale, with_lse=True)
    got = out32.cpu().numpy().astype(np.float64).reshape(R, D)
    gl = lse.cpu().numpy().astype(np.float64)
    empty = ~np.isfinite(ref_lse)
    assert empty.sum() == 18                  # rows 5-7 of 8, 6 heads each
    assert np.all(gl[empty] == -np.inf) and not got[empty].any()
    scale = np.abs(ref_out).max()
    assert np.abs(got - ref_out).max() <= 2e-6 * scale
    assert np.all(np.abs(gl[~empty] - ref_lse[~empty]) <= 2e-6 * np.maximum(1.0, np.abs(ref_lse[~empty])))


@pytest.mark.parametrize("cut", [1, 100, 255])
def test_cross_rank_merge(orc, cut):
    """Two groups of splits standing for two ranks, each combined with its LSE
    and merged by the LSE rule on the host, give the one-pass combine and the
    oracle's output at the parity bar."""
    announce("cross-rank merge c3", cut)
    w, p, ws = _c3_workspace()
    R, D, S = w.q_rows * w.num_heads, w.head_dim, p.num_splits
    acc, mx, sm = ws
    parts = []
    for lo, hi in ((0, cut), (cut, S)):
        o32 = torch.empty(R * D, dtype=torch.float32, device=gu.DEV)
        l32 = torch.empty(R, dtype=torch.float32, device=gu.DEV)
        part = (acc[lo:hi], mx[lo:hi], sm[lo:hi])         # workspace is [S][rows](...)
        pa.paged_attn_combine_fp32_lse(part, hi - lo, R, D, w.v_scale, out32=o32, lse=l32)
        parts.append((o32, l32))
    full = torch.empty(R * D, dtype=torch.float32, device=gu.DEV)
    pa.paged_attn_combine_fp32_lse(ws, S, R, D, w.v_scale, out32=full)
    torch.cuda.synchronize()
    merged, _ = lse_merge([(o.cpu().numpy().astype(np.float64).reshape(R, D),
                            l.cpu().numpy().astype(np.float64)) for o, l in parts])
    one = full.cpu().numpy().astype(np.float64).reshape(R, D)
    assert np.abs(merged - one).max() <= 4e-6 * np.abs(one).max()
    ref = orc.dense_workload(w).reshape(R, D)
    gu.assert_parity(merged.astype(np.float16), ref, f"cross-rank merge cut {cut}")


# ---------------------------------------------------------------------------
# batches of independent requests (q up to 16, row chunks, Hkv > 1)
# ---------------------------------------------------------------------------

BATCHES = [
    # (ctxs, q_rows, H, Hkv, D, page, row_lens, splits)
    ([700, 130, 1], 16, 6, 1, 256, 96, None, 0),
    ([300, 64, 517, 1000], 4, 8, 2, 128, 64, [[300, 0, 299, 1], [64, 64, 0, 63],
                                                [517, 500, 1, 2], [0, 0, 0, 0]], 3),
    ([2500, 900], 12, 4, 1, 256, 848, None, 5),
    ([129, 64, 200], 16, 6, 2, 256, 1, None, 2),
    # long splits over pages of 1000 (span 1728: block references moved in place
    # inside a page and looked up across page edges)
    ([5000, 2900, 640], 8, 6, 1, 256, 1000, None, 8),
]


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("case", range(len(BATCHES)))
def test_batch_small(orc, case, kernel):
    ctxs, qr, H, Hkv, D, page, lens, splits = BATCHES[case]
    w = wl.make_dense_batch(f"batch{case}", 0xBA7C0 + case, ctxs=ctxs, q_rows=qr,
                            num_heads=H, num_kv_heads=Hkv, head_dim=D, page_size=page,
                            sigma=1.2, k_scale=0.45, v_scale=1.6, row_lens=lens,
                            num_splits=splits)
    announce("batch", case, ctxs, qr, H, Hkv, D, page, kernel)
    got = gu.run_batch(w, kernel)
    gu.assert_parity(got, gu.oracle_batch(orc, w), f"batch{case}/{kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
def test_batch_matches_single_requests(kernel):
    """The batch entry shares its splits over the requests by length: one span
    T for the batch, request b's unit taking ceil(L_b / T) consecutive splits.
    The split index it writes equals the host's re-derivation of that rule,
    and each unit's partials (numerators where the split is not empty) are
    bit-identical to the single-request entry's with splits of T tokens (whose
    further splits are empty)."""
    w = wl.make_dense_batch("bsingle", 0xB51, ctxs=[1000, 300, 770], q_rows=8, num_heads=6,
                            num_kv_heads=1, head_dim=256, page_size=96, sigma=1.0,
                            k_scale=0.5, v_scale=1.5, max_blocks=12)
    lens = w.row_lens.copy()
    lens[2] = [770, 700, 0, 3, 770, 500, 769, 1]
    w = dataclasses.replace(w, row_lens=lens)
    S = 9
    announce("batch vs single", kernel)
    _, bp, (bacc, bmx, bsm, bidx) = gu.run_batch(w, kernel, splits=S, return_ws=True)
    T, index = gu.ragged_plan(w.row_lens, w.cap, w.num_kv_heads, bp.num_splits,
                              bp.tokens_per_split)
    assert np.array_equal(bidx, index), (bidx, index)
    R = w.q_rows * w.num_heads
    for b in range(w.batch):
        r = dataclasses.replace(w.request(b), max_tokens=w.cap)
        d = gu.dense_to_dev(r)
        p = pa.plan(w.cap, R // w.num_kv_heads, w.num_kv_heads, w.head_dim, w.page_size,
                    kernel=kernel)
        p.tokens_per_split = T
        p.num_splits = -(-w.cap // T)
        ws = pa.make_workspace(p, R, w.head_dim, gu.DEV)
        pa.paged_attn_verify_e4m3(d.q, d.k, d.v, d.table, d.lens, w.cap, w.sm_scale,
                                  w.k_scale, p, ws)
        torch.cuda.synchronize()
        acc, mx, sm = (t.cpu().numpy() for t in ws)
        s0, s1 = index[b], index[b + 1]
        n = s1 - s0
        assert np.array_equal(bmx[s0:s1], mx[:n]) and np.array_equal(bsm[s0:s1], sm[:n]), b
        # numerators are compared where the split is not empty (sum != 0): an
        # empty split's numerator is not written
        live = sm[:n] != 0
        assert np.array_equal(bacc[s0:s1][live], acc[:n][live]), b
        assert np.all(mx[n:] == -np.inf) and not sm[n:].any(), b


@pytest.mark.parametrize("kernel", KERNELS)
def test_batch_combine_lse(orc, kernel):
    """The batch combine for a merge across ranks: its FP16 output is
    bit-identical to the plain batch combine's; its FP32 output and base-2 LSE
    match the FP64 oracle merge of each unit's own FP32 partials (the split
    index the verify wrote); rows of length zero give LSE -inf and zeros."""
    w = wl.make_dense_batch("blse", 0xB15E, ctxs=[1000, 300, 770], q_rows=4, num_heads=12,
                            num_kv_heads=2, head_dim=128, page_size=96, sigma=1.0,
                            k_scale=0.5, v_scale=1.5, max_blocks=12)
    lens = w.row_lens.copy()
    lens[1] = [300, 0, 250, 1]
    w = dataclasses.replace(w, row_lens=lens)
    announce("batch combine lse", kernel)
    _, p, ws = gu.run_batch(w, kernel, splits=11, return_ws=True)
    dev_ws = tuple(torch.from_numpy(x).to(gu.DEV) for x in ws)
    B, Q, H, Hkv, D = w.batch, w.q_rows, w.num_heads, w.num_kv_heads, w.head_dim
    G = H // Hkv
    rows = B * Q * H
    out16 = torch.empty(rows * D, dtype=torch.float16, device=gu.DEV)
    ref16 = torch.empty(rows * D, dtype=torch.float16, device=gu.DEV)
    out32 = torch.empty(rows * D, dtype=torch.float32, device=gu.DEV)
    lse = torch.empty(rows, dtype=torch.float32, device=gu.DEV)
    pa.paged_attn_combine_batch_fp32(dev_ws, p, B, Q, H, Hkv, D, w.v_scale, ref16)
    pa.paged_attn_combine_batch_fp32_lse(dev_ws, p, B, Q, H, Hkv, D, w.v_scale, out=out16,
                                         out32=out32, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out16, ref16)
    acc, mx, sm, index = ws
    got = out32.cpu().numpy().astype(np.float64).reshape(B, Q, H, D)
    gl = lse.cpu().numpy().astype(np.float64).reshape(B, Q, H)
    for b in range(B):
        for g in range(Hkv):
            u = b * Hkv + g
            s0, s1 = int(index[u]), int(index[u + 1])
            ref_out, ref_lse = orc.combine(acc[s0:s1], mx[s0:s1], sm[s0:s1], w.v_scale,
                                           with_lse=True)
            for ru in range(Q * G):
                i, h = ru // G, g * G + ru % G
                if not np.isfinite(ref_lse[ru]):
                    assert gl[b, i, h] == -np.inf and not got[b, i, h].any(), (b, i, h)
                    continue
                scale = max(np.abs(ref_out[ru]).max(), 1e-30)
                assert np.abs(got[b, i, h] - ref_out[ru]).max() <= 2e-6 * scale, (b, i, h)
                assert abs(gl[b, i, h] - ref_lse[ru]) <= 2e-6 * max(1.0, abs(ref_lse[ru])), (b, i, h)
    assert np.isinf(gl[1, 1]).all() and not got[1, 1].any()      # the zero-length row


def test_batch_config(orc):
    """The named batch configuration (8 requests, q16, contexts 4K-32K) at full
    size, the MFMA kernel in the benchmark's plan."""
    w = wl.cached("batch")
    announce("batch config", w.name)
    got = gu.run_batch(w, "mfma")
    gu.assert_parity(got, gu.oracle_batch(orc, w, nthreads=16), "batch config")


# ---------------------------------------------------------------------------
# E4M3 cache write
# ---------------------------------------------------------------------------

def _write_and_compare(orc, k_bits, v_bits, slots, k0, v0, ks, vs, view=None):
    """GPU write into (a view of) device copies of k0/v0; returns host pools."""
    kd = torch.from_numpy(k0).to(gu.DEV)
    vd = torch.from_numpy(v0).to(gu.DEV)
    kv_k, kv_v = (kd, vd) if view is None else (view(kd), view(vd))
    pa.paged_attn_cache_write_e4m3(gu.fp16_tensor(k_bits).to(gu.DEV),
                                   gu.fp16_tensor(v_bits).to(gu.DEV),
                                   torch.from_numpy(slots).to(gu.DEV), kv_k, kv_v, ks, vs)
    torch.cuda.synchronize()
    return kd.cpu().numpy(), vd.cpu().numpy()


@pytest.mark.parametrize("scale", [1.0, 0.37, 2.25, 2.0 ** -7, 0.0625, 3.0, 61.0, 1000.0,
                                   2.0 ** -120, 2.0 ** 125])
def test_cache_write_every_fp16_value(orc, scale):
    """Every FP16 bit pattern, written with k_scale = scale (and v_scale =
    1/scale), gives the oracle encoder's byte for the FP32 quotient, bit for bit.
    The last two scales put one of the pair outside [2^-110, 2^126], where the
    writer divides without the reciprocal."""
    announce("cache write all fp16", scale)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(4096, 1, 16)
    T, P, ps = 4096, 256, 16                 # 16-byte token rows: the pool's stride rule
    slots = np.arange(T, dtype=np.int64)
    k0 = np.zeros((P, ps, 1, 16), np.uint8)
    v0 = np.zeros((P, ps, 1, 16), np.uint8)
    ks, vs = np.float32(scale), np.float32(1.0 / scale)
    gk, gv = _write_and_compare(orc, bits, bits, slots, k0, v0, ks, vs)
    rk, rv = orc.cache_write(bits, bits, slots, k0, v0, ks, vs)
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


def test_cache_write_slots_and_specials(orc):
    """Random tokens with specials into shuffled slots of a pool with random
    bytes: skipped (-1) and out-of-range slots write nothing, everything else is
    bit-exact with the oracle."""
    rng = np.random.Generator(np.random.PCG64(0xCA11))
    T, Hkv, D, P, ps = 300, 2, 128, 24, 16
    vals = (rng.standard_normal((T, Hkv, D)) * 30.0).astype(np.float16)
    vals[0, 0, :8] = [0.0, -0.0, np.nan, np.inf, -np.inf, 60000.0, 2 ** -16, -448.0]
    slots = rng.permutation(P * ps)[:T].astype(np.int64)
    slots[[3, 77, 150]] = -1
    slots[[4, 200]] = P * ps + 5                      # past the pool: skipped on the device
    k0 = rng.integers(0, 256, (P, ps, Hkv, D), dtype=np.uint8)
    v0 = rng.integers(0, 256, (P, ps, Hkv, D), dtype=np.uint8)
    announce("cache write slots")
    gk, gv = _write_and_compare(orc, vals.view(np.uint16), (-vals).view(np.uint16), slots,
                                k0, v0, np.float32(0.45), np.float32(1.6))
    ok_slots = np.where(slots >= P * ps, -1, slots)
    rk, rv = orc.cache_write(vals.view(np.uint16), (-vals).view(np.uint16), ok_slots, k0, v0,
                             np.float32(0.45), np.float32(1.6))
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


def test_cache_write_strided_view(orc):
    """A packed allocation (K of one pool interleaved with other data): only the
    view's bytes change, and they match the oracle on the view."""
    rng = np.random.Generator(np.random.PCG64(0xCA12))
    T, Hkv, D, P, ps = 40, 1, 256, 6, 8
    vals = (rng.standard_normal((T, Hkv, D)) * 4.0).astype(np.float16)
    slots = rng.permutation(P * ps)[:T].astype(np.int64)
    big_k = rng.integers(0, 256, (P, ps, 2, Hkv, D), dtype=np.uint8)   # [.., plane, ..]
    big_v = rng.integers(0, 256, (P, ps, 2, Hkv, D), dtype=np.uint8)
    announce("cache write strided view")
    gk, gv = _write_and_compare(orc, vals.view(np.uint16), vals.view(np.uint16), slots, big_k,
                                big_v, np.float32(0.5), np.float32(0.5),
                                view=lambda t: t[:, :, 1])
    rk, rv = orc.cache_write(vals.view(np.uint16), vals.view(np.uint16), slots,
                             np.ascontiguousarray(big_k[:, :, 1]),
                             np.ascontiguousarray(big_v[:, :, 1]), np.float32(0.5),
                             np.float32(0.5))
    assert np.array_equal(gk[:, :, 1], rk) and np.array_equal(gv[:, :, 1], rv)
    assert np.array_equal(gk[:, :, 0], big_k[:, :, 0]) and np.array_equal(gv[:, :, 0], big_v[:, :, 0])
