"""GPU parity over seeded random shapes, through the C ABI, against the oracle.

Each case draws a shape the boundary accepts -- grouped heads, head dim 128 or
256, page sizes from 1 token to several thousand (multiples of 32 and not),
contexts up to a few thousand tokens, causal or arbitrary row lengths (zero,
past the capacity, negative), planner-chosen or requested split counts, and
for the MFMA kernel the plan's row chunk or a forced one of 16, 32 or 48 rows -- for
the dense verify of one request, the ragged batch of independent requests and
the sparse verify over selected blocks and over selected token ids, and checks the output against the FP64
oracle at the usual bar (rel-L2 <= 5e-4, max-abs <= 4x the FP16 rounding
floor).  The draws are fixed by their seeds, so a failing case is reproduced by
its index.
"""

import numpy as np
import pytest

from fp8_kv_paged_attn_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

KERNELS = ["mfma", "simple"]
PAGES = [1, 3, 16, 31, 32, 33, 64, 100, 160, 288, 517, 1000, 2048]


def announce(*what):
    print("[case]", *what, flush=True)


def _lens(rng, q_rows: int, ctx: int):
    """None (causal: row i sees ctx - q_rows + 1 + i) or arbitrary lengths."""
    if rng.random() < 0.5:
        return None
    lens = [int(x) for x in rng.integers(-5, ctx + 30, size=q_rows)]
    for i in range(q_rows):
        if rng.random() < 0.2:
            lens[i] = 0
    return lens


def _group_and_rows(rng, max_rows: int, max_q: int):
    G = int(rng.choice([1, 2, 3, 4, 6, 8, 12]))
    q_rows = int(rng.integers(1, max(1, min(max_q, max_rows // G)) + 1))
    return G, q_rows


def dense_case(i: int):
    rng = np.random.default_rng(0xD5E0 + i)
    D = int(rng.choice([128, 256]))
    Hkv = int(rng.choice([1, 2, 4]))
    G, q_rows = _group_and_rows(rng, 48, 8)
    page = int(rng.choice(PAGES))
    ctx = int(rng.integers(q_rows, 3000))
    npages = -(-ctx // page)
    splits = 0 if rng.random() < 0.4 else int(rng.integers(1, 13))
    return dict(q_rows=q_rows, num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D, ctx=ctx,
                page_size=page, pool_pages=npages + int(rng.integers(0, 4)),
                sigma=float(rng.uniform(0.5, 2.0)), k_scale=float(rng.uniform(0.2, 3.0)),
                v_scale=float(rng.uniform(0.2, 3.0)), row_lens=_lens(rng, q_rows, ctx),
                num_splits=splits, poison_tail=bool(rng.random() < 0.5))


def batch_case(i: int):
    rng = np.random.default_rng(0xBA70 + i)
    D = int(rng.choice([128, 256]))
    Hkv = int(rng.choice([1, 2]))
    G, q_rows = _group_and_rows(rng, 96, 16)
    page = int(rng.choice(PAGES))
    B = int(rng.integers(1, 7))
    ctxs = [int(x) for x in rng.integers(1, 2500, size=B)]
    lens = None
    if rng.random() < 0.5:
        lens = [_lens(rng, q_rows, c) or [c] * q_rows for c in ctxs]
    splits = 0 if rng.random() < 0.4 else int(rng.integers(1, 41))
    return dict(ctxs=ctxs, q_rows=q_rows, num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                page_size=page, sigma=float(rng.uniform(0.5, 2.0)),
                k_scale=float(rng.uniform(0.2, 3.0)), v_scale=float(rng.uniform(0.2, 3.0)),
                row_lens=lens, num_splits=splits)


def qsa_case(i: int):
    rng = np.random.default_rng(0x05A0 + i)
    D = int(rng.choice([128, 256]))
    Hkv = int(rng.choice([1, 2]))
    G, q_rows = _group_and_rows(rng, 48, 8)
    page = int(rng.choice([16, 32, 48, 64, 100]))
    nblk = int(rng.integers(2, 40))
    ctx = nblk * page - int(rng.integers(0, page))
    topk = int(rng.integers(1, -(-ctx // page) + 1))
    B = int(rng.integers(1, 5))
    lens = None
    if rng.random() < 0.5:
        lens = np.stack([np.array(_lens(rng, q_rows, ctx) or [ctx] * q_rows, np.int64)
                         for _ in range(B)])
    splits = 0 if rng.random() < 0.4 else int(rng.integers(1, 9))
    return dict(batch=B, q_rows=q_rows, num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                ctx=ctx, page_size=page, topk=topk, k_scale=float(rng.uniform(0.2, 3.0)),
                v_scale=float(rng.uniform(0.2, 3.0)), num_splits=splits, row_lens=lens)


def tokens_case(i: int):
    rng = np.random.default_rng(0x70C0 + i)
    D = int(rng.choice([128, 256]))
    Hkv = int(rng.choice([1, 2]))
    G, q_rows = _group_and_rows(rng, 48, 8)
    page = int(rng.choice([16, 32, 48, 64, 100, 333]))
    ctx = int(rng.integers(q_rows + 8, 3000))
    num_empty = int(rng.integers(0, 5))
    num_sel = int(rng.integers(q_rows + num_empty + 1, min(ctx, 2500) + 1))
    B = int(rng.integers(1, 4))
    lens = None
    if rng.random() < 0.5:
        lens = np.stack([np.array(_lens(rng, q_rows, ctx) or [ctx] * q_rows, np.int64)
                         for _ in range(B)])
    splits = 0 if rng.random() < 0.4 else int(rng.integers(1, 9))
    return dict(batch=B, q_rows=q_rows, num_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                ctx=ctx, page_size=page, num_sel=num_sel, k_scale=float(rng.uniform(0.2, 3.0)),
                v_scale=float(rng.uniform(0.2, 3.0)), num_empty=num_empty, num_splits=splits,
                row_lens=lens)


N_DENSE, N_BATCH, N_QSA, N_TOKENS = 80, 40, 40, 24


def row_chunk(kind: int, i: int, kernel: str):
    """Rows per MFMA workgroup for case i: the plan's (None) or 16, 32 or 48
    forced (drawn from a stream of its own, so the shapes do not change)."""
    if kernel != "mfma":
        return None
    r = int(np.random.default_rng(0xC4C0 + 1000 * kind + i).choice([0, 16, 32, 48]))
    return r or None


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("i", range(N_DENSE))
def test_random_dense(orc, i, kernel):
    args = dense_case(i)
    announce("random dense", i, kernel, {k: v for k, v in args.items() if k != "row_lens"},
             "lens", args["row_lens"])
    w = wl.make_dense(f"rnd_dense{i}", 0xD5E000 + i, **args)
    rpw = row_chunk(0, i, kernel)
    announce("rows per workgroup", rpw)
    got = gu.run_dense(w, kernel, rows_per_workgroup=rpw)
    gu.assert_parity(got, orc.dense_workload(w), f"random dense {i}/{kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("i", range(N_BATCH))
def test_random_batch(orc, i, kernel):
    args = batch_case(i)
    announce("random batch", i, kernel, {k: v for k, v in args.items() if k != "row_lens"},
             "lens", args["row_lens"])
    w = wl.make_dense_batch(f"rnd_batch{i}", 0xBA7000 + i, **args)
    got = gu.run_batch(w, kernel)
    gu.assert_parity(got, gu.oracle_batch(orc, w), f"random batch {i}/{kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("i", range(N_QSA))
def test_random_qsa(orc, i, kernel):
    args = qsa_case(i)
    announce("random qsa", i, kernel, {k: v for k, v in args.items() if k != "row_lens"},
             "lens", None if args["row_lens"] is None else args["row_lens"].tolist())
    w = wl.make_qsa(f"rnd_qsa{i}", 0x05A000 + i, **args)
    rpw = row_chunk(1, i, kernel)
    announce("rows per workgroup", rpw)
    got = gu.run_qsa(w, kernel, rows_per_workgroup=rpw)
    gu.assert_parity(got, orc.qsa_workload(w), f"random qsa {i}/{kernel}")


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("i", range(N_TOKENS))
def test_random_qsa_tokens(orc, i, kernel):
    args = tokens_case(i)
    announce("random qsa tokens", i, kernel,
             {k: v for k, v in args.items() if k != "row_lens"},
             "lens", None if args["row_lens"] is None else args["row_lens"].tolist())
    w = wl.make_qsa_tokens(f"rnd_tok{i}", 0x70C000 + i, **args)
    rpw = row_chunk(2, i, kernel)
    announce("rows per workgroup", rpw)
    got = gu.run_qsa_tokens(w, kernel, rows_per_workgroup=rpw)
    gu.assert_parity(got, orc.qsa_tokens_workload(w), f"random qsa tokens {i}/{kernel}")
