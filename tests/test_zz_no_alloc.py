"""The allocation-free dense entry (paged_attn_verify_noalloc_e4m3): its split
partials live in the library's fixed per-device scratch array.  Through the C
ABI it must give exactly what the workspace entry gives (verify +
combine, same kernels), on two calls in a row, the second smaller than the
first, so that the second reads only what it wrote over the first call's
leftovers; and a plan larger than the scratch is refused before any work."""

import ctypes

import numpy as np
import pytest
import torch

import fp8_kv_paged_attn_amd as pa
from fp8_kv_paged_attn_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _noalloc(w, d, p):
    out = torch.full((w.q_rows, w.num_heads, w.head_dim), float("nan"), dtype=torch.float16,
                     device=gu.DEV)
    pa.paged_attn_verify_noalloc_e4m3(d.q, d.k, d.v, d.table, d.lens, w.max_tokens, w.sm_scale,
                                      w.k_scale, w.v_scale, p, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_noalloc_matches_workspace_entry_two_calls(orc):
    gu.require_gpu()
    big = wl.cached("c2_64k")                 # 256 splits x 48 rows x D256: 12.7 MB
    small = wl.make_dense("noalloc_small", 0xA110C, q_rows=3, num_heads=6, num_kv_heads=1,
                          head_dim=256, ctx=5000, page_size=1616, pool_pages=8, sigma=1.5,
                          k_scale=0.37, v_scale=1.9, row_lens=[4998, 5000, 0])
    for w in (big, small):
        print(f"[case] noalloc {w.name}", flush=True)
        d = gu.dense_to_dev(w)
        p = gu.dense_plan(w)
        got = _noalloc(w, d, p)
        ref = gu.run_dense(w, d=d)
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), w.name
        gu.assert_parity(got, orc.dense_workload(w), f"noalloc {w.name}")


def test_noalloc_refuses_a_plan_past_the_scratch():
    gu.require_gpu()
    w = wl.make_dense("noalloc_big", 0xA110D, q_rows=8, num_heads=6, num_kv_heads=1,
                      head_dim=256, ctx=1 << 15, page_size=4096, pool_pages=10, sigma=1.0,
                      k_scale=1.0, v_scale=1.0)
    p = pa.plan(w.max_tokens, 48, 1, 256, w.page_size, splits=512)
    need = p.num_splits * 48 * (256 + 2) * 4
    assert need > pa.NOALLOC_SCRATCH_BYTES
    d = gu.dense_to_dev(w)
    out = torch.zeros((8, 6, 256), dtype=torch.float16, device=gu.DEV)
    with pytest.raises(RuntimeError, match="-8|scratch"):
        pa.paged_attn_verify_noalloc_e4m3(d.q, d.k, d.v, d.table, d.lens, w.max_tokens,
                                          w.sm_scale, w.k_scale, w.v_scale, p, out)
    torch.cuda.synchronize()
    assert not out.cpu().numpy().any(), "a refused call wrote its output"
