"""Seeded synthetic workloads for the verify-attention path.

This module only draws random numbers and lays them out in the shapes the
attention path consumes (query rows, paged E4M3 K/V pools, block tables,
per-row lengths, block selections).  It holds none of the attention
arithmetic: no decoding of E4M3 bytes, no dot products, no softmax.

The one numeric transform here is the quantisation of the drawn K/V values
into E4M3 bytes.  That is the job of the KV-cache writer upstream of the
attention path (the vLLM PR "Qwen4Exp: fp8_e4m3 main KV cache on the QSA
path" writes the cache with ``reshape_and_cache_flash`` and per-tensor
scales, Changes section); it is written here from the format definition
(OCP E4M3FN: bias 7, no infinities, 0x7F/0xFF NaN, max 448) with
round-to-nearest-even and saturation, by float32 bit manipulation.  The
oracle has its own, independently written encoder; a CPU test checks the two
agree on every float32 midpoint and on dense sweeps.

Random numbers: splitmix64 (Steele, Lea and Flood 2014, the published
finaliser constants) drives a counter-based stream; Box-Muller turns pairs of
53-bit uniforms into normals.  Every array is a pure function of
(base seed, tag, index), so any slice can be regenerated without the rest.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)

# splitmix64 constants, as published with the generator.
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_MIX1 = np.uint64(0xBF58476D1CE4E5B9)
_MIX2 = np.uint64(0x94D049BB133111EB)

E4M3_NAN = 0x7F


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.uint64, copy=True)
    z ^= z >> np.uint64(30)
    z *= _MIX1
    z ^= z >> np.uint64(27)
    z *= _MIX2
    z ^= z >> np.uint64(31)
    return z


def splitmix64_scalar(x: int) -> int:
    """splitmix64 finaliser of (x + golden) on one 64-bit integer."""
    z = (x + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    return z ^ (z >> 31)


def substream_seed(base: int, tag: str) -> int:
    """Seed of the named sub-stream (Q, K, V, permutation, selection...)."""
    h = 0
    for ch in tag.encode():
        h = splitmix64_scalar(h ^ ch)
    return splitmix64_scalar(base ^ h)


def uniform_u64(seed: int, start: int, count: int) -> np.ndarray:
    """count raw 64-bit outputs of the counter-based stream, from index start."""
    with np.errstate(over="ignore"):
        ctr = np.arange(start, start + count, dtype=np.uint64)
        z = np.uint64(seed) + (ctr + np.uint64(1)) * _GOLDEN
        return _mix64(z)


def uniform01(seed: int, start: int, count: int) -> np.ndarray:
    """Uniforms in (0, 1): (top 53 bits + 0.5) / 2^53, never 0 or 1."""
    u = uniform_u64(seed, start, count) >> np.uint64(11)
    return (u.astype(np.float64) + 0.5) * (1.0 / 9007199254740992.0)


def normal(seed: int, start: int, count: int, sigma: float = 1.0) -> np.ndarray:
    """count N(0, sigma) draws (Box-Muller over consecutive uniform pairs)."""
    if count == 0:
        return np.zeros(0, np.float64)
    first = start - (start % 2)
    npairs = (start + count - first + 1) // 2
    u = uniform01(seed, first, 2 * npairs)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    z = np.empty(2 * npairs, np.float64)
    z[0::2] = r * np.cos(2.0 * np.pi * u2)
    z[1::2] = r * np.sin(2.0 * np.pi * u2)
    off = start - first
    return z[off:off + count] * sigma


def randint(seed: int, start: int, count: int, hi: int) -> np.ndarray:
    """count integers uniform in [0, hi) (multiply-shift on 32-bit draws)."""
    u = (uniform_u64(seed, start, count) >> np.uint64(32)).astype(np.uint64)
    return ((u * np.uint64(hi)) >> np.uint64(32)).astype(np.int64)


def permutation(seed: int, n: int) -> np.ndarray:
    """Seeded Fisher-Yates permutation of range(n)."""
    p = np.arange(n, dtype=np.int64)
    if n <= 1:
        return p
    r = uniform01(seed, 0, n)
    for i in range(n - 1, 0, -1):
        j = int(r[i] * (i + 1))
        p[i], p[j] = p[j], p[i]
    return p


def quantize_e4m3(x: np.ndarray) -> np.ndarray:
    """float32 values -> E4M3FN bytes, round-to-nearest-even, saturating.

    |x| is clamped to 448 first, so overflow saturates to 0x7E/0xFE; NaN gives
    0x7F.  Normals round the float32 significand from 23 to 3 bits (ties to
    even); values below 2^-6 are counted in units of 2^-9 and rounded with
    numpy's rint (ties to even).
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    sign = ((bits >> np.uint32(24)) & np.uint32(0x80)).astype(np.uint8)
    nan = np.isnan(x)
    a = np.where(nan, np.float32(0.0), np.minimum(np.abs(x), np.float32(448.0)))
    abits = a.view(np.uint32).astype(np.uint64)
    # normal range: RNE on the low 20 bits of the float32 pattern
    lsb = (abits >> np.uint64(20)) & np.uint64(1)
    rounded = (abits + np.uint64(0x7FFFF) + lsb) >> np.uint64(20)
    normal_code = rounded.astype(np.int64) - ((127 - 7) << 3)
    sub_code = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)
    code = np.where(a >= np.float32(2.0 ** -6), normal_code, sub_code)
    code = np.clip(code, 0, 0x7E).astype(np.uint8)
    out = code | sign
    out = np.where(nan, np.uint8(E4M3_NAN), out).astype(np.uint8)
    return out


def _fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bfloat16 bit patterns (via float32, round-to-nearest-even)."""
    f = np.asarray(x, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    lsb = (f >> np.uint64(16)) & np.uint64(1)
    return ((f + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------


@dataclasses.dataclass
class DenseWorkload:
    """One verify request over a paged E4M3 pool (the dense path)."""

    name: str
    q_bits: np.ndarray         # uint16 fp16 bits, [q_rows][num_heads][head_dim]
    k_pool: np.ndarray         # uint8, [num_pages][page_size][num_kv_heads][head_dim]
    v_pool: np.ndarray         # uint8, same shape
    block_table: np.ndarray    # int32 [num_entries]
    row_lens: np.ndarray       # int32 [q_rows]
    max_tokens: int
    q_rows: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    sm_scale: float
    k_scale: float
    v_scale: float
    num_splits: int = 0        # 0: planner decides

    @property
    def num_rows(self) -> int:
        return self.q_rows * self.num_heads

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes: longest visible prefix x heads x D x 2."""
        lmax = int(np.clip(self.row_lens, 0, self.max_tokens).max(initial=0))
        return lmax * self.num_kv_heads * self.head_dim * 2


@dataclasses.dataclass
class QsaWorkload:
    """A batch of sparse verify requests over selected blocks."""

    name: str
    q_bits: np.ndarray         # uint16 bf16 bits, [batch][q_rows][num_heads][head_dim]
    k_pool: np.ndarray         # uint8, [num_pages][page_size][num_kv_heads][head_dim]
    v_pool: np.ndarray
    block_table: np.ndarray    # int32 [batch][max_blocks]
    sel_blocks: np.ndarray     # int32 [batch][num_kv_heads][topk], -1 = empty
    row_lens: np.ndarray       # int32 [batch][q_rows]
    batch: int
    q_rows: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_blocks: int
    topk: int
    sm_scale: float
    k_scale: float
    v_scale: float
    num_splits: int = 0

    @property
    def num_rows(self) -> int:
        return self.batch * self.q_rows * self.num_heads

    def kv_bytes(self) -> int:
        """Algorithmic bytes: selected tokens x D x 2 per (request, KV head)."""
        nsel = int((self.sel_blocks >= 0).sum())
        return nsel * self.page_size * self.head_dim * 2


def _fill_plane(pool: np.ndarray, seed: int, pages: List[int], page_size: int,
                sigma: float, scale: float, outlier_ch: Optional[np.ndarray],
                outlier_mult: float) -> None:
    """Quantise N(0, sigma)/scale into the given physical pages (in order)."""
    _, psz, hkv, d = pool.shape
    per_page = psz * hkv * d
    for idx, p in enumerate(pages):
        x = normal(seed, idx * per_page, per_page, sigma).reshape(psz, hkv, d)
        if outlier_ch is not None:
            x[:, :, outlier_ch] *= outlier_mult
        pool[p] = quantize_e4m3((x / scale).astype(np.float32))


def make_dense(name: str, seed: int, *, q_rows: int, num_heads: int,
               num_kv_heads: int, head_dim: int, ctx: int, page_size: int,
               pool_pages: int, sigma: float, k_scale: float, v_scale: float,
               row_lens: Optional[List[int]] = None, num_splits: int = 0,
               shuffle: bool = True, outlier_channels: int = 0,
               outlier_mult: float = 8.0, null_page_nan: bool = False,
               pad_table_to: int = 0, poison_unused: bool = True,
               poison_tail: bool = False,
               sm_scale: Optional[float] = None) -> DenseWorkload:
    """Build a seeded single-request verify workload.

    Logical pages are placed on a seeded sample of physical pages.  Unused
    physical pages hold random bytes including NaN codes when poison_unused.
    null_page_nan reserves physical page 0 as a NaN-filled null block and pads
    the block table with it up to pad_table_to entries.  poison_tail fills the
    unused tail of the last real page with the NaN byte.
    """
    n_log = -(-ctx // page_size)
    first_phys = 1 if null_page_nan else 0
    assert pool_pages - first_phys >= n_log
    sq = substream_seed(seed, "Q")
    sk = substream_seed(seed, "K")
    sv = substream_seed(seed, "V")
    sp = substream_seed(seed, "perm")
    sj = substream_seed(seed, "junk")
    so = substream_seed(seed, "outlier")

    q = normal(sq, 0, q_rows * num_heads * head_dim, 1.0)
    q_bits = _fp16_bits(q).reshape(q_rows, num_heads, head_dim)

    cand = np.arange(first_phys, pool_pages)
    if shuffle:
        cand = cand[permutation(sp, cand.size)]
    phys = [int(p) for p in cand[:n_log]]

    shape = (pool_pages, page_size, num_kv_heads, head_dim)
    k_pool = np.zeros(shape, np.uint8)
    v_pool = np.zeros(shape, np.uint8)
    if poison_unused:
        # random bytes (NaN codes included) in every page; real pages are
        # overwritten below.  numpy's seeded PCG64 is enough for filler.
        rng = np.random.Generator(np.random.PCG64(sj))
        k_pool[...] = rng.integers(0, 256, size=shape, dtype=np.uint8)
        v_pool[...] = rng.integers(0, 256, size=shape, dtype=np.uint8)
        k_pool.reshape(-1)[::7] = E4M3_NAN
        v_pool.reshape(-1)[::7] = E4M3_NAN
    outl = None
    if outlier_channels:
        outl = np.sort(permutation(so, head_dim)[:outlier_channels])
    _fill_plane(k_pool, sk, phys, page_size, sigma, k_scale, outl, outlier_mult)
    _fill_plane(v_pool, sv, phys, page_size, sigma, v_scale, None, 1.0)
    if null_page_nan:
        k_pool[0] = E4M3_NAN
        v_pool[0] = E4M3_NAN
    if poison_tail:
        tail = ctx - (n_log - 1) * page_size
        k_pool[phys[-1], tail:] = E4M3_NAN
        v_pool[phys[-1], tail:] = E4M3_NAN

    table = list(phys)
    if pad_table_to:
        table += [0] * (pad_table_to - len(table))
    if row_lens is None:
        row_lens = [ctx - q_rows + i + 1 for i in range(q_rows)]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return DenseWorkload(
        name=name, q_bits=q_bits, k_pool=k_pool, v_pool=v_pool,
        block_table=np.asarray(table, np.int32),
        row_lens=np.asarray(row_lens, np.int32), max_tokens=ctx,
        q_rows=q_rows, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, page_size=page_size, sm_scale=float(np.float32(sm_scale)),
        k_scale=float(np.float32(k_scale)), v_scale=float(np.float32(v_scale)),
        num_splits=num_splits)


@dataclasses.dataclass
class DenseBatchWorkload:
    """A batch of independent dense verify requests sharing one pool."""

    name: str
    q_bits: np.ndarray         # uint16 fp16 bits, [batch][q_rows][num_heads][head_dim]
    k_pool: np.ndarray         # uint8, [num_pages][page_size][num_kv_heads][head_dim]
    v_pool: np.ndarray
    block_table: np.ndarray    # int32 [batch][max_blocks]
    row_lens: np.ndarray       # int32 [batch][q_rows]
    batch: int
    q_rows: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_blocks: int
    sm_scale: float
    k_scale: float
    v_scale: float
    num_splits: int = 0

    @property
    def num_rows(self) -> int:
        return self.batch * self.q_rows * self.num_heads

    @property
    def cap(self) -> int:
        return self.max_blocks * self.page_size

    def request(self, b: int) -> DenseWorkload:
        """Request b as a single-request workload over the shared pool."""
        return DenseWorkload(
            name=f"{self.name}[{b}]", q_bits=self.q_bits[b], k_pool=self.k_pool,
            v_pool=self.v_pool, block_table=self.block_table[b], row_lens=self.row_lens[b],
            max_tokens=self.cap, q_rows=self.q_rows, num_heads=self.num_heads,
            num_kv_heads=self.num_kv_heads, head_dim=self.head_dim, page_size=self.page_size,
            sm_scale=self.sm_scale, k_scale=self.k_scale, v_scale=self.v_scale)

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes: per request, longest visible prefix x heads x D x 2."""
        lmax = np.clip(self.row_lens, 0, self.cap).max(axis=1)
        return int(lmax.sum()) * self.num_kv_heads * self.head_dim * 2


def make_dense_batch(name: str, seed: int, *, ctxs: List[int], q_rows: int, num_heads: int,
                     num_kv_heads: int, head_dim: int, page_size: int, sigma: float,
                     k_scale: float, v_scale: float, max_blocks: Optional[int] = None,
                     row_lens: Optional[List[List[int]]] = None,
                     num_splits: int = 0) -> DenseBatchWorkload:
    """A batch of requests of context ctxs[b], each built like make_dense (its
    own seeded sub-stream), their pages concatenated into one pool.  Table rows
    are padded to max_blocks with the request's first page; rows see
    ctx - q_rows + 1 + i tokens unless row_lens is given."""
    B = len(ctxs)
    need = [-(-c // page_size) for c in ctxs]
    max_blocks = max_blocks or max(need)
    assert max_blocks >= max(need)
    reqs = []
    for b, c in enumerate(ctxs):
        lens = None if row_lens is None else row_lens[b]
        reqs.append(make_dense(f"{name}_{b}", substream_seed(seed, f"req{b}"), q_rows=q_rows,
                               num_heads=num_heads, num_kv_heads=num_kv_heads,
                               head_dim=head_dim, ctx=c, page_size=page_size,
                               pool_pages=need[b] + 1, sigma=sigma, k_scale=k_scale,
                               v_scale=v_scale, row_lens=lens))
    k_pool = np.concatenate([r.k_pool for r in reqs])
    v_pool = np.concatenate([r.v_pool for r in reqs])
    table = np.zeros((B, max_blocks), np.int32)
    base = 0
    for b, r in enumerate(reqs):
        t = r.block_table.astype(np.int64) + base
        table[b, :t.size] = t
        table[b, t.size:] = t[0]
        base += r.k_pool.shape[0]
    return DenseBatchWorkload(
        name=name, q_bits=np.stack([r.q_bits for r in reqs]), k_pool=k_pool, v_pool=v_pool,
        block_table=table, row_lens=np.stack([r.row_lens for r in reqs]).astype(np.int32),
        batch=B, q_rows=q_rows, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, page_size=page_size, max_blocks=max_blocks,
        sm_scale=reqs[0].sm_scale, k_scale=reqs[0].k_scale, v_scale=reqs[0].v_scale,
        num_splits=num_splits)


def config_c4_tokens() -> QsaTokensWorkload:
    """The QSA batch of c4 with a token-id selection: 2048 ids per (request, KV
    head), the newest 4 tokens always included, 32 of them -1."""
    return make_qsa_tokens("c4tok_qsa_b16_q4_h24_kv2_d128_r2048", BASE_SEED + 6, batch=16,
                           q_rows=4, num_heads=24, num_kv_heads=2, head_dim=128, ctx=32768,
                           page_size=64, num_sel=2048, num_empty=32, k_scale=0.5,
                           v_scale=2.0)


def config_batch() -> DenseBatchWorkload:
    """Independent-request batch: 8 requests, q16 rows, H6/Hkv1/D256, E4M3 pages of
    3296 tokens, contexts 4K..32K (mixed lengths), k 0.37, v 1.9."""
    ctxs = [32768, 4096, 16384, 24576, 8192, 28672, 12288, 20480]
    return make_dense_batch("batch_b8_q16_h6_kv1_d256_4k-32k", BASE_SEED + 5, ctxs=ctxs,
                            q_rows=16, num_heads=6, num_kv_heads=1, head_dim=256,
                            page_size=3296, sigma=1.5, k_scale=0.37, v_scale=1.9)


def make_qsa(name: str, seed: int, *, batch: int, q_rows: int, num_heads: int,
             num_kv_heads: int, head_dim: int, ctx: int, page_size: int,
             topk: int, k_scale: float, v_scale: float, sigma: float = 1.0,
             num_splits: int = 0, poison_unselected: bool = True,
             sm_scale: Optional[float] = None,
             row_lens: Optional[np.ndarray] = None) -> QsaWorkload:
    """Build a seeded sparse-selection verify batch.

    Each request owns ctx/page_size logical blocks placed at seeded physical
    pages.  Each (request, KV head) selects topk distinct blocks: the block
    holding the newest token plus topk-1 drawn from the others, stored in a
    shuffled order.  Only selected pages hold real data; with
    poison_unselected every other page is filled with the NaN byte.
    """
    nblk = -(-ctx // page_size)
    pool_pages = batch * nblk
    sq = substream_seed(seed, "Q")
    sk = substream_seed(seed, "K")
    sv = substream_seed(seed, "V")
    sp = substream_seed(seed, "perm")
    ss = substream_seed(seed, "sel")

    q = normal(sq, 0, batch * q_rows * num_heads * head_dim, 1.0)
    q_bits = _bf16_bits(q).reshape(batch, q_rows, num_heads, head_dim)

    perm = permutation(sp, pool_pages)
    table = perm.reshape(batch, nblk).astype(np.int32)

    sel = np.empty((batch, num_kv_heads, topk), np.int32)
    for b in range(batch):
        for g in range(num_kv_heads):
            sub = substream_seed(ss, f"{b}/{g}")
            others = permutation(sub, nblk - 1)[: topk - 1]
            chosen = np.concatenate([others, [nblk - 1]])
            order = permutation(substream_seed(sub, "order"), topk)
            sel[b, g] = chosen[order]

    shape = (pool_pages, page_size, num_kv_heads, head_dim)
    fill = E4M3_NAN if poison_unselected else 0
    k_pool = np.full(shape, fill, np.uint8)
    v_pool = np.full(shape, fill, np.uint8)
    per_head = page_size * head_dim
    for b in range(batch):
        for g in range(num_kv_heads):
            for blk in sel[b, g]:
                p = int(table[b, blk])
                base = ((b * nblk + int(blk)) * num_kv_heads + g) * per_head
                xk = normal(sk, base, per_head, sigma).reshape(page_size, head_dim)
                xv = normal(sv, base, per_head, sigma).reshape(page_size, head_dim)
                k_pool[p, :, g, :] = quantize_e4m3((xk / k_scale).astype(np.float32))
                v_pool[p, :, g, :] = quantize_e4m3((xv / v_scale).astype(np.float32))
    if row_lens is None:
        row_lens = np.array([[ctx - q_rows + i + 1 for i in range(q_rows)]] * batch, np.int32)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return QsaWorkload(
        name=name, q_bits=q_bits, k_pool=k_pool, v_pool=v_pool, block_table=table,
        sel_blocks=sel, row_lens=np.asarray(row_lens, np.int32), batch=batch,
        q_rows=q_rows, num_heads=num_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, page_size=page_size, max_blocks=nblk, topk=topk,
        sm_scale=float(np.float32(sm_scale)), k_scale=float(np.float32(k_scale)),
        v_scale=float(np.float32(v_scale)), num_splits=num_splits)


@dataclasses.dataclass
class QsaTokensWorkload:
    """A batch of sparse verify requests over selected token ids (-1 = empty)."""

    name: str
    q_bits: np.ndarray         # uint16 bf16 bits, [batch][q_rows][num_heads][head_dim]
    k_pool: np.ndarray         # uint8, [num_pages][page_size][num_kv_heads][head_dim]
    v_pool: np.ndarray
    block_table: np.ndarray    # int32 [batch][max_blocks]
    sel_tokens: np.ndarray     # int32 [batch][num_kv_heads][num_sel], -1 = empty
    row_lens: np.ndarray       # int32 [batch][q_rows]
    batch: int
    q_rows: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_blocks: int
    num_sel: int
    sm_scale: float
    k_scale: float
    v_scale: float
    num_splits: int = 0

    @property
    def num_rows(self) -> int:
        return self.batch * self.q_rows * self.num_heads

    def kv_bytes(self) -> int:
        """Algorithmic bytes: selected token ids x D x 2 per (request, KV head)."""
        return int((self.sel_tokens >= 0).sum()) * self.head_dim * 2


def tokens_from_blocks(w: QsaWorkload) -> np.ndarray:
    """The token-id form of a block selection: block s becomes ids s*page ..
    s*page + page - 1 in list order; an empty block slot becomes page -1s."""
    ps = w.page_size
    out = np.full((w.batch, w.num_kv_heads, w.topk * ps), -1, np.int32)
    for b in range(w.batch):
        for g in range(w.num_kv_heads):
            for j, blk in enumerate(w.sel_blocks[b, g]):
                if blk >= 0:
                    out[b, g, j * ps:(j + 1) * ps] = np.arange(blk * ps, (blk + 1) * ps)
    return out


def make_qsa_tokens(name: str, seed: int, *, batch: int, q_rows: int, num_heads: int,
                    num_kv_heads: int, head_dim: int, ctx: int, page_size: int, num_sel: int,
                    k_scale: float, v_scale: float, num_empty: int = 0, sigma: float = 1.0,
                    num_splits: int = 0,
                    row_lens: Optional[np.ndarray] = None) -> QsaTokensWorkload:
    """Build a seeded token-id selection batch.  Every block of every request
    holds data (a block selection of all blocks, unpoisoned); each (request, KV
    head) selects the newest q_rows tokens plus num_sel - q_rows - num_empty
    distinct older ones, with num_empty -1 entries, in a shuffled order."""
    nblk = -(-ctx // page_size)
    base = make_qsa(name, seed, batch=batch, q_rows=q_rows, num_heads=num_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, ctx=ctx, page_size=page_size,
                    topk=nblk, k_scale=k_scale, v_scale=v_scale, sigma=sigma,
                    poison_unselected=False, row_lens=row_lens)
    ss = substream_seed(seed, "tokens")
    n_old = num_sel - q_rows - num_empty
    assert 0 <= n_old <= ctx - q_rows
    sel = np.empty((batch, num_kv_heads, num_sel), np.int32)
    for b in range(batch):
        for g in range(num_kv_heads):
            sub = substream_seed(ss, f"{b}/{g}")
            old = permutation(sub, ctx - q_rows)[:n_old]
            new = np.arange(ctx - q_rows, ctx)
            chosen = np.concatenate([old, new, np.full(num_empty, -1)])
            sel[b, g] = chosen[permutation(substream_seed(sub, "order"), num_sel)]
    return QsaTokensWorkload(
        name=name, q_bits=base.q_bits, k_pool=base.k_pool, v_pool=base.v_pool,
        block_table=base.block_table, sel_tokens=sel, row_lens=base.row_lens, batch=batch,
        q_rows=q_rows, num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        page_size=page_size, max_blocks=nblk, num_sel=num_sel, sm_scale=base.sm_scale,
        k_scale=base.k_scale, v_scale=base.v_scale, num_splits=num_splits)


# ---------------------------------------------------------------------------
# The five named configurations
# ---------------------------------------------------------------------------

BASE_SEED = 0xC0DE0000


def config_c0() -> DenseWorkload:
    """q2, H6/Hkv1/D256, ctx 2048, page 800 in a shuffled 6-page pool, 4 splits."""
    return make_dense("c0_q2_ctx2048_page800", BASE_SEED + 0, q_rows=2, num_heads=6,
                      num_kv_heads=1, head_dim=256, ctx=2048, page_size=800,
                      pool_pages=6, sigma=1.0, k_scale=1.0, v_scale=1.0, num_splits=4)


def config_c1() -> DenseWorkload:
    """q8, ctx 8192, page 3296 in a 64-page pool, k=0.37 v=1.9, N(0,1.5)."""
    return make_dense("c1_q8_ctx8192_page3296", BASE_SEED + 1, q_rows=8, num_heads=6,
                      num_kv_heads=1, head_dim=256, ctx=8192, page_size=3296,
                      pool_pages=64, sigma=1.5, k_scale=0.37, v_scale=1.9)


def config_c2(ctx: int) -> DenseWorkload:
    """C1's shape at 16K-128K; pool of 2x pages; 3 K channels x8 larger."""
    n_log = -(-ctx // 3296)
    return make_dense(f"c2_q8_ctx{ctx}_page3296", BASE_SEED + 2, q_rows=8, num_heads=6,
                      num_kv_heads=1, head_dim=256, ctx=ctx, page_size=3296,
                      pool_pages=2 * n_log, sigma=1.5, k_scale=0.37, v_scale=1.9,
                      outlier_channels=math.ceil(0.01 * 256), poison_unused=False)


def config_c3() -> DenseWorkload:
    """q8, ctx 262144, page 3456, rows 5-7 length 0, NaN null page 0, k=0.5 v=2.25."""
    ctx, page = 262144, 3456
    n_log = -(-ctx // page)                       # 76 real pages
    lens = [ctx - 5 + i + 1 for i in range(5)] + [0, 0, 0]
    return make_dense("c3_q8_ctx262144_page3456", BASE_SEED + 3, q_rows=8, num_heads=6,
                      num_kv_heads=1, head_dim=256, ctx=ctx, page_size=page,
                      pool_pages=n_log + 1, sigma=1.0, k_scale=0.5, v_scale=2.25,
                      row_lens=lens, null_page_nan=True,
                      pad_table_to=-(-n_log // 8) * 8, poison_unused=False,
                      poison_tail=True, shuffle=True)


def config_c4() -> QsaWorkload:
    """QSA: B16, q4, H24/Hkv2/D128, ctx 32768 in 64-token blocks, top-32."""
    return make_qsa("c4_qsa_b16_q4_h24_kv2_d128_top32", BASE_SEED + 4, batch=16,
                    q_rows=4, num_heads=24, num_kv_heads=2, head_dim=128, ctx=32768,
                    page_size=64, topk=32, k_scale=0.5, v_scale=2.0)


def tiny_dense(seed: int, **kw) -> DenseWorkload:
    """Small dense case for fast CPU/GPU checks (defaults overridable)."""
    args = dict(q_rows=2, num_heads=4, num_kv_heads=2, head_dim=128, ctx=300,
                page_size=48, pool_pages=9, sigma=1.0, k_scale=0.75, v_scale=1.25)
    args.update(kw)
    return make_dense(f"tiny_dense_{seed:x}", seed, **args)


_CACHE: Dict[str, object] = {}


def cached(name: str):
    """The named configuration, generated once per process."""
    if name not in _CACHE:
        _CACHE[name] = CONFIGS[name]()
    return _CACHE[name]


CONFIGS: Dict[str, object] = {
    "c0": config_c0,
    "c1": config_c1,
    "c2_16k": lambda: config_c2(16384),
    "c2_32k": lambda: config_c2(32768),
    "c2_64k": lambda: config_c2(65536),
    "c2_128k": lambda: config_c2(131072),
    "c3": config_c3,
    "c4": config_c4,
    "batch": config_batch,
    "c4tok": config_c4_tokens,
}
