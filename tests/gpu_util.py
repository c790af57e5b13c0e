"""Helpers for the GPU tests: move seeded workloads to the device, run the
library through its C ABI, and apply the acceptance bar.

Acceptance (FP16 output against the FP64 oracle o):
  rel-L2  ||gpu - o|| / ||o||              <= 5e-4
  max-abs max |gpu - o|                    <= 4 x max |fp16(o) - o|
The second bound is relative to the FP16 output-rounding floor, as the design
note "DFlash2 E4M3 attention with FP32 state" bounds its errors ("Rebuilt
operator results": relative to the FP16 output-rounding floor, not only an
aggregate tolerance)."""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

import fp8_kv_paged_attn_amd as pa

DEV = torch.device("cuda:0")


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device (cuda:0)")


def fp16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16)


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


@dataclasses.dataclass
class DenseDev:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    table: torch.Tensor
    lens: torch.Tensor


def dense_to_dev(w) -> DenseDev:
    return DenseDev(fp16_tensor(w.q_bits).to(DEV), torch.from_numpy(w.k_pool).to(DEV),
                    torch.from_numpy(w.v_pool).to(DEV),
                    torch.from_numpy(w.block_table.astype(np.int32)).to(DEV),
                    torch.from_numpy(w.row_lens.astype(np.int32)).to(DEV))


def dense_plan(w, kernel="auto", splits: Optional[int] = None):
    G = w.num_heads // w.num_kv_heads
    s = w.num_splits if splits is None else splits
    return pa.plan(w.max_tokens, w.q_rows * G, w.num_kv_heads, w.head_dim, w.page_size,
                   splits=s, kernel=kernel)


def run_dense(w, kernel="auto", splits: Optional[int] = None, d: Optional[DenseDev] = None,
              k=None, v=None, return_ws=False, rows_per_workgroup: Optional[int] = None):
    d = d or dense_to_dev(w)
    p = dense_plan(w, kernel, splits)
    if rows_per_workgroup is not None:
        p.rows_per_workgroup = rows_per_workgroup
    ws = pa.make_workspace(p, w.q_rows * w.num_heads, w.head_dim, DEV)
    out = pa.verify(d.q, d.k if k is None else k, d.v if v is None else v, d.table, d.lens,
                    w.max_tokens, sm_scale=w.sm_scale, k_scale=w.k_scale, v_scale=w.v_scale,
                    p=p, ws=ws)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if return_ws:
        return res, p, tuple(t.cpu().numpy() for t in ws)
    return res


def run_batch(w, kernel="auto", splits: Optional[int] = None, return_ws=False):
    """A DenseBatchWorkload through paged_attn_verify_batch_e4m3 + combine."""
    q = fp16_tensor(w.q_bits).to(DEV)
    k = torch.from_numpy(w.k_pool).to(DEV)
    v = torch.from_numpy(w.v_pool).to(DEV)
    bt = torch.from_numpy(w.block_table.astype(np.int32)).to(DEV)
    lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(DEV)
    G = w.num_heads // w.num_kv_heads
    s = w.num_splits if splits is None else splits
    p = pa.plan(w.cap, w.q_rows * G, w.batch * w.num_kv_heads, w.head_dim, w.page_size,
                "batch", splits=s, kernel=kernel)
    ws = pa.make_workspace(p, w.batch * w.q_rows * w.num_heads, w.head_dim, DEV)
    out = pa.verify_batch(q, k, v, bt, lens, sm_scale=w.sm_scale, k_scale=w.k_scale,
                          v_scale=w.v_scale, p=p, ws=ws)
    torch.cuda.synchronize()
    if return_ws:
        return out.cpu().numpy(), p, tuple(t.cpu().numpy() for t in ws)
    return out.cpu().numpy()


def ragged_plan(row_lens, cap: int, num_kv_heads: int, num_splits: int, tcap: int):
    """The split layout a ragged batch's kernels derive on the device, worked
    out on the host from the same rule: span T and split index [units + 1]."""
    L = np.clip(np.asarray(row_lens, np.int64), 0, cap).max(axis=1)
    U = L.size * num_kv_heads
    total = int(L.sum()) * num_kv_heads
    T = tcap
    if num_splits > U:
        t = -(-total // (num_splits - U))
        T = max(64, min(-(-t // 64) * 64, tcap))
    per_unit = np.repeat(-(-L // T), num_kv_heads)
    index = np.concatenate([[0], np.cumsum(per_unit)]).astype(np.int64)
    return T, index


def oracle_batch(orc, w, nthreads=1) -> np.ndarray:
    """The oracle request by request (each over the shared pool, capped at the
    table width)."""
    return np.stack([orc.dense_workload(w.request(b), nthreads=nthreads)
                     for b in range(w.batch)])


def run_qsa(w, kernel="auto", splits: Optional[int] = None, return_ws=False,
            rows_per_workgroup: Optional[int] = None):
    q = bf16_tensor(w.q_bits).to(DEV)
    k = torch.from_numpy(w.k_pool).to(DEV)
    v = torch.from_numpy(w.v_pool).to(DEV)
    bt = torch.from_numpy(w.block_table.astype(np.int32)).to(DEV)
    sel = torch.from_numpy(w.sel_blocks.astype(np.int32)).to(DEV)
    lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(DEV)
    G = w.num_heads // w.num_kv_heads
    s = w.num_splits if splits is None else splits
    p = pa.plan(w.topk * w.page_size, w.q_rows * G, w.batch * w.num_kv_heads, w.head_dim,
                w.page_size, "blocks", splits=s, kernel=kernel)
    if rows_per_workgroup is not None:
        p.rows_per_workgroup = rows_per_workgroup
    ws = pa.make_workspace(p, w.batch * w.q_rows * w.num_heads, w.head_dim, DEV)
    out = pa.qsa_verify(q, k, v, bt, sel, lens, sm_scale=w.sm_scale, k_scale=w.k_scale,
                        v_scale=w.v_scale, p=p, ws=ws)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if return_ws:
        return res, p, tuple(t.cpu().numpy() for t in ws)
    return res


def run_qsa_tokens(w, kernel="auto", splits: Optional[int] = None, k_pool=None, v_pool=None,
                   rows_per_workgroup: Optional[int] = None):
    """Token-id selection batch through qsa_sparse_verify_tokens_e4m3 + combine."""
    q = bf16_tensor(w.q_bits).to(DEV)
    k = torch.from_numpy(w.k_pool if k_pool is None else k_pool).to(DEV)
    v = torch.from_numpy(w.v_pool if v_pool is None else v_pool).to(DEV)
    bt = torch.from_numpy(w.block_table.astype(np.int32)).to(DEV)
    sel = torch.from_numpy(w.sel_tokens.astype(np.int32)).to(DEV)
    lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(DEV)
    G = w.num_heads // w.num_kv_heads
    s = w.num_splits if splits is None else splits
    p = pa.plan(w.num_sel, w.q_rows * G, w.batch * w.num_kv_heads, w.head_dim, w.page_size,
                "tokens", splits=s, kernel=kernel)
    if rows_per_workgroup is not None:
        p.rows_per_workgroup = rows_per_workgroup
    out = pa.qsa_verify_tokens(q, k, v, bt, sel, lens, sm_scale=w.sm_scale, k_scale=w.k_scale,
                               v_scale=w.v_scale, p=p)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def metrics(gpu: np.ndarray, ref: np.ndarray) -> dict:
    g = gpu.astype(np.float64)
    err = g - ref
    rounded = ref.astype(np.float16).astype(np.float64)
    nref = float(np.linalg.norm(ref))
    floor_abs = float(np.abs(rounded - ref).max(initial=0.0))
    return dict(
        rel_l2=float(np.linalg.norm(err)) / nref if nref > 0 else float(np.linalg.norm(err)),
        floor_rel_l2=float(np.linalg.norm(rounded - ref)) / nref if nref > 0 else 0.0,
        max_abs=float(np.abs(err).max(initial=0.0)),
        floor_abs=floor_abs,
        finite=bool(np.all(np.isfinite(g))),
    )


def assert_parity(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    m = metrics(gpu, ref)
    print(f"[parity] {what}: rel_l2={m['rel_l2']:.3e} (floor {m['floor_rel_l2']:.3e}) "
          f"max_abs={m['max_abs']:.3e} (4x floor {4 * m['floor_abs']:.3e})", flush=True)
    assert m["finite"], f"{what}: non-finite output"
    assert m["rel_l2"] <= 5e-4, f"{what}: rel-L2 {m['rel_l2']:.3e} > 5e-4"
    assert m["max_abs"] <= 4 * m["floor_abs"], \
        f"{what}: max-abs {m['max_abs']:.3e} > 4 x floor {m['floor_abs']:.3e}"
    return m
