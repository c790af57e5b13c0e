"""The seeded input generator: determinism, shapes, and its test-data E4M3
quantiser against the oracle's independently written encoder."""

import dataclasses

import numpy as np

from fp8_kv_paged_attn_amd import workloads as wl
from tests.oracle_pins import _encoder_sweep


def test_splitmix64_published_values():
    # splitmix64 from state 0: the first outputs of the published generator.
    state, outs = 0, []
    for _ in range(3):
        outs.append(wl.splitmix64_scalar(state))
        state = (state + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    assert outs == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    # the vectorised counter stream agrees with the scalar form
    v = wl.uniform_u64(0, 0, 3)
    assert [int(x) for x in v] == outs


def test_quantiser_matches_oracle_encoder(orc):
    x = _encoder_sweep()
    x = np.concatenate([x, np.array([448.0, 460.0, 1e5, -1e5, 0.0, -0.0], np.float32)])
    assert np.array_equal(wl.quantize_e4m3(x), orc.e4m3_encode(x.astype(np.float64)))
    rng = np.random.default_rng(1)
    y = (rng.standard_normal(200000) * rng.choice([1e-3, 1.0, 50.0, 300.0], 200000)).astype(np.float32)
    assert np.array_equal(wl.quantize_e4m3(y), orc.e4m3_encode(y.astype(np.float64)))
    assert wl.quantize_e4m3(np.array([np.nan], np.float32))[0] == 0x7F


def test_normals_are_normal():
    z = wl.normal(123, 0, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    # any slice regenerates identically
    assert np.array_equal(wl.normal(123, 1001, 77), z[1001:1078])
    assert np.array_equal(wl.normal(123, 1000, 77), z[1000:1077])


def test_generator_deterministic_and_shaped():
    a = wl.config_c0()
    b = wl.config_c0()
    assert np.array_equal(a.k_pool, b.k_pool) and np.array_equal(a.q_bits, b.q_bits)
    assert a.k_pool.shape == (6, 800, 1, 256) and a.block_table.size == 3
    assert list(a.row_lens) == [2047, 2048] and a.num_splits == 4
    assert len(set(a.block_table.tolist())) == 3


def test_c3_layout():
    # only the table/lengths logic, on a reduced page so the test stays fast
    w = wl.make_dense("c3_small", 3, q_rows=8, num_heads=6, num_kv_heads=1, head_dim=16,
                      ctx=1000, page_size=96, pool_pages=12, sigma=1.0, k_scale=0.5,
                      v_scale=2.25, row_lens=[996, 997, 998, 999, 1000, 0, 0, 0],
                      null_page_nan=True, pad_table_to=16, poison_unused=False,
                      poison_tail=True)
    assert (w.k_pool[0] == 0x7F).all() and (w.v_pool[0] == 0x7F).all()
    assert list(w.block_table[11:]) == [0] * 5 and 0 not in list(w.block_table[:11])
    last = w.block_table[10]
    assert (w.k_pool[last, 1000 - 960:] == 0x7F).all()
    assert w.kv_bytes() == 1000 * 16 * 2


def test_qsa_selection_shape():
    w = wl.make_qsa("q", 5, batch=3, q_rows=4, num_heads=8, num_kv_heads=2, head_dim=16,
                    ctx=640, page_size=64, topk=4, k_scale=0.5, v_scale=2.0)
    assert w.sel_blocks.shape == (3, 2, 4)
    for b in range(3):
        for g in range(2):
            s = w.sel_blocks[b, g]
            assert 9 in s and len(set(s.tolist())) == 4
    assert w.kv_bytes() == 3 * 2 * 4 * 64 * 16 * 2


def test_token_selection_shape():
    w = wl.make_qsa_tokens("t", 6, batch=2, q_rows=3, num_heads=4, num_kv_heads=2,
                           head_dim=16, ctx=300, page_size=32, num_sel=40, num_empty=5,
                           k_scale=0.5, v_scale=2.0)
    assert w.sel_tokens.shape == (2, 2, 40) and w.max_blocks == 10
    for b in range(2):
        for g in range(2):
            s = w.sel_tokens[b, g]
            ids = s[s >= 0]
            assert (s == -1).sum() == 5 and len(set(ids.tolist())) == 35
            assert ids.max() < 300 and set(range(297, 300)) <= set(ids.tolist())
    # every page of every request holds data (no NaN poison)
    assert not (w.k_pool == 0x7F).all(axis=(1, 2, 3)).any()
    assert w.kv_bytes() == 2 * 2 * 35 * 16 * 2


def test_tokens_from_blocks():
    q = wl.make_qsa("q", 7, batch=2, q_rows=2, num_heads=4, num_kv_heads=2, head_dim=16,
                    ctx=256, page_size=16, topk=3, k_scale=0.5, v_scale=2.0)
    sel = q.sel_blocks.copy()
    sel[1, 0, 1] = -1
    q = dataclasses.replace(q, sel_blocks=sel)
    t = wl.tokens_from_blocks(q)
    assert t.shape == (2, 2, 48)
    assert list(t[0, 0, :16]) == list(range(sel[0, 0, 0] * 16, sel[0, 0, 0] * 16 + 16))
    assert (t[1, 0, 16:32] == -1).all()
