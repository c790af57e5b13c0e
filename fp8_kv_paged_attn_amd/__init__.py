"""Multi-row verify attention over a paged FP8-E4M3 KV cache, for MI355X.

Thin ctypes binding over ``libpaged_attn_e4m3.so`` (HIP, gfx950), whose C ABI
is ``include/paged_attn_e4m3.h``.  This module only checks devices and dtypes
and marshals pointers; every step of the computation runs in the library's
kernels.  PyTorch provides device memory and the current stream.  There is no
CPU fallback: without the built library every call raises.

Entry points (same names as the C ABI):
  plan(...)                      split planner (pure host)
  paged_attn_verify_e4m3(...)    dense verify, writes FP32 split partials
  paged_attn_combine_fp32(...)   merges partials into FP16 rows
  qsa_sparse_verify_e4m3(...)    sparse verify over selected blocks
  qsa_sparse_verify_tokens_e4m3(...)  sparse verify over selected token ids
and the conveniences ``verify``, ``verify_batch``, ``qsa_verify`` and
``qsa_verify_tokens`` (verify + combine).
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_attn_e4m3.so")
ABI_VERSION = 3

PA_KERNEL = {"auto": 0, "simple": 1, "mfma": 2}
PA_SELECTION = {"dense": 0, "blocks": 1, "tokens": 2, "batch": 3}


class PaKvPool(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("page_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64), ("num_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32)]


class PaPlan(ctypes.Structure):
    _fields_ = [("num_splits", ctypes.c_int32), ("tokens_per_split", ctypes.c_int32),
                ("kernel", ctypes.c_int32), ("max_tokens", ctypes.c_int32),
                ("rows_per_kv_unit", ctypes.c_int32), ("num_kv_units", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("selection", ctypes.c_int32), ("ws_acc_bytes", ctypes.c_int64),
                ("ws_stat_bytes", ctypes.c_int64), ("ws_index_bytes", ctypes.c_int64),
                ("rows_per_workgroup", ctypes.c_int32)]

    def __repr__(self):
        return (f"PaPlan(splits={self.num_splits}, tokens_per_split={self.tokens_per_split}, "
                f"kernel={self.kernel}, max_tokens={self.max_tokens}, "
                f"rows={self.rows_per_kv_unit}, units={self.num_kv_units}, "
                f"rows_per_workgroup={self.rows_per_workgroup})")


class PaWorkspace(ctypes.Structure):
    _fields_ = [("acc", ctypes.c_void_p), ("max", ctypes.c_void_p), ("sum", ctypes.c_void_p),
                ("acc_bytes", ctypes.c_int64), ("stat_bytes", ctypes.c_int64),
                ("index", ctypes.c_void_p), ("index_bytes", ctypes.c_int64)]


EXPORTS = ("paged_attn_abi_version", "paged_attn_build_id", "paged_attn_status_string",
           "paged_attn_plan",
           "paged_attn_verify_e4m3", "paged_attn_combine_fp32", "qsa_sparse_verify_e4m3",
           "paged_attn_timer_arm", "paged_attn_timer_read", "paged_attn_stream_read_probe",
           "paged_attn_combine_fp32_lse", "paged_attn_verify_batch_e4m3",
           "paged_attn_cache_write_e4m3", "qsa_sparse_verify_tokens_e4m3",
           "paged_attn_verify_noalloc_e4m3", "paged_attn_combine_batch_fp32",
           "paged_attn_combine_batch_fp32_lse")

_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it was not built, has another ABI revision,
    or was built from sources other than the ones beside this module."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m fp8_kv_paged_attn_amd.build` (there is no CPU fallback)")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, p, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    L.paged_attn_abi_version.argtypes = []
    L.paged_attn_abi_version.restype = i32
    L.paged_attn_build_id.argtypes = []
    L.paged_attn_build_id.restype = ctypes.c_char_p
    L.paged_attn_status_string.argtypes = [i32]
    L.paged_attn_status_string.restype = ctypes.c_char_p
    L.paged_attn_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(PaPlan)]
    L.paged_attn_plan.restype = i32
    L.paged_attn_verify_e4m3.argtypes = [p, ctypes.POINTER(PaKvPool), p, i32, p, i32, i32, i32,
                                         i32, i32, f32, f32, ctypes.POINTER(PaPlan),
                                         ctypes.POINTER(PaWorkspace), p]
    L.paged_attn_verify_e4m3.restype = i32
    L.paged_attn_combine_fp32.argtypes = [p, p, p, i32, i32, i32, f32, p, p]
    L.paged_attn_combine_fp32.restype = i32
    L.paged_attn_verify_noalloc_e4m3.argtypes = [p, ctypes.POINTER(PaKvPool), p, i32, p, i32,
                                                 i32, i32, i32, i32, f32, f32, f32,
                                                 ctypes.POINTER(PaPlan), p, p]
    L.paged_attn_verify_noalloc_e4m3.restype = i32
    L.paged_attn_verify_batch_e4m3.argtypes = [p, ctypes.POINTER(PaKvPool), p, i32, p, i32, i32,
                                               i32, i32, i32, f32, f32, ctypes.POINTER(PaPlan),
                                               ctypes.POINTER(PaWorkspace), p]
    L.paged_attn_verify_batch_e4m3.restype = i32
    L.paged_attn_combine_batch_fp32.argtypes = [ctypes.POINTER(PaWorkspace),
                                                ctypes.POINTER(PaPlan), i32, i32, i32, i32, i32,
                                                f32, p, p]
    L.paged_attn_combine_batch_fp32.restype = i32
    L.paged_attn_combine_batch_fp32_lse.argtypes = [ctypes.POINTER(PaWorkspace),
                                                    ctypes.POINTER(PaPlan), i32, i32, i32, i32,
                                                    i32, f32, p, p, p, p]
    L.paged_attn_combine_batch_fp32_lse.restype = i32
    L.paged_attn_cache_write_e4m3.argtypes = [p, p, i64, i32, i32, p, ctypes.POINTER(PaKvPool),
                                              f32, f32, p]
    L.paged_attn_cache_write_e4m3.restype = i32
    L.paged_attn_combine_fp32_lse.argtypes = [p, p, p, i32, i32, i32, f32, p, p, p, p]
    L.paged_attn_combine_fp32_lse.restype = i32
    L.qsa_sparse_verify_e4m3.argtypes = [p, ctypes.POINTER(PaKvPool), p, i32, p, i32, p, i32,
                                         i32, i32, i32, i32, f32, f32, ctypes.POINTER(PaPlan),
                                         ctypes.POINTER(PaWorkspace), p]
    L.qsa_sparse_verify_e4m3.restype = i32
    L.qsa_sparse_verify_tokens_e4m3.argtypes = L.qsa_sparse_verify_e4m3.argtypes
    L.qsa_sparse_verify_tokens_e4m3.restype = i32
    L.paged_attn_timer_arm.argtypes = [i32]
    L.paged_attn_timer_arm.restype = i32
    L.paged_attn_timer_read.argtypes = [ctypes.POINTER(ctypes.c_float), i32,
                                        ctypes.POINTER(ctypes.c_int32)]
    L.paged_attn_timer_read.restype = i32
    L.paged_attn_stream_read_probe.argtypes = [p, i64, p, p]
    L.paged_attn_stream_read_probe.restype = i32
    ver = L.paged_attn_abi_version()
    if ver != ABI_VERSION:
        raise RuntimeError(f"libpaged_attn_e4m3 ABI revision {ver}, this binding needs "
                           f"{ABI_VERSION}: rebuild the library")
    from . import build as _build

    built, here = L.paged_attn_build_id().decode(), _build.source_hash()
    if built != here:
        raise RuntimeError(f"libpaged_attn_e4m3 was built from other sources (build id {built}, "
                           f"sources here {here}): rebuild the library")
    _LIB = L
    return L


def build_id() -> str:
    """Source hash compiled into the loaded library."""
    return lib().paged_attn_build_id().decode()


TIMER_MAX_LAUNCHES = 1024


def timer_arm(n: int) -> None:
    """Time the kernels of the next `n` verify launches (0 disarms)."""
    _check(lib().paged_attn_timer_arm(int(n)), "paged_attn_timer_arm")


def timer_read() -> list:
    """Kernel times in ms of the launches timed since timer_arm, in launch
    order (waits for them); disarms."""
    ms = (ctypes.c_float * TIMER_MAX_LAUNCHES)()
    n = ctypes.c_int32(0)
    _check(lib().paged_attn_timer_read(ms, TIMER_MAX_LAUNCHES, ctypes.byref(n)),
           "paged_attn_timer_read")
    return [float(ms[i]) for i in range(min(n.value, TIMER_MAX_LAUNCHES))]


def stream_read_probe(buf, sink) -> None:
    """Read all of buf (a contiguous device tensor, size a multiple of 16 bytes)
    once on the current stream; sink is a device tensor of at least 4 bytes."""
    nbytes = buf.numel() * buf.element_size()
    if not buf.is_contiguous() or sink.device != buf.device or sink.numel() * sink.element_size() < 4:
        raise ValueError("buf must be contiguous and sink a 4-byte tensor on its device")
    _check(lib().paged_attn_stream_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(),
                                              _stream(buf.device)), "paged_attn_stream_read_probe")


def status_string(rc: int) -> str:
    return lib().paged_attn_status_string(int(rc)).decode()


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed: {status_string(rc)} ({rc})")


def plan(max_tokens: int, rows_per_kv_unit: int, num_kv_units: int, head_dim: int,
         page_size: int, selection: str = "dense", num_cus: int = 0, splits: int = 0,
         kernel: str = "auto") -> PaPlan:
    """Split plan (host integer arithmetic in the library; num_cus = 0 takes the
    current device's compute-unit count)."""
    out = PaPlan()
    _check(lib().paged_attn_plan(int(max_tokens), int(rows_per_kv_unit), int(num_kv_units),
                                 int(head_dim), int(page_size), PA_SELECTION[selection],
                                 int(num_cus), int(splits), ctypes.byref(out)),
           "paged_attn_plan")
    out.kernel = PA_KERNEL[kernel]
    return out


# ---------------------------------------------------------------------------
# Tensor marshalling
# ---------------------------------------------------------------------------


def _torch():
    import torch

    return torch


def _scale(x, name: str) -> float:
    """Scales are host scalars: k_scale is folded into the logit scale on the
    host and v_scale passed by value (vLLM PR "Qwen4Exp: fp8_e4m3 main KV cache
    on the QSA path", review thread on host-side KV scales), so reading a
    device tensor would cost a synchronisation and break graph capture.  A
    Python number or a one-element CPU tensor is accepted; a tensor on any
    other device is refused before anything is enqueued."""
    torch = _torch()
    if isinstance(x, torch.Tensor):
        if x.device.type != "cpu":
            raise ValueError(f"{name} must be a host scalar (a float or a CPU tensor), "
                             f"not a tensor on {x.device}: the library takes scales by value")
        if x.numel() != 1:
            raise ValueError(f"{name} must have one element")
        x = x.item()
    x = float(x)
    if not math.isfinite(x):
        raise ValueError(f"{name} must be finite")
    return x


def _pool(k_pool, v_pool, device) -> PaKvPool:
    torch = _torch()
    for t, n in ((k_pool, "k_pool"), (v_pool, "v_pool")):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{n} must hold E4M3 bytes (uint8 or float8_e4m3fn)")
        if t.device != device:
            raise ValueError(f"{n} is on {t.device}, the query is on {device}")
        if t.dim() != 4 or t.stride(3) != 1:
            raise ValueError(f"{n} must be [pages][page_size][kv_heads][head_dim], head_dim contiguous")
    if k_pool.shape != v_pool.shape or k_pool.stride() != v_pool.stride():
        raise ValueError("k_pool and v_pool must have the same shape and strides")
    return PaKvPool(k_pool.data_ptr(), v_pool.data_ptr(), k_pool.stride(0), k_pool.stride(1),
                    k_pool.stride(2), k_pool.shape[0], k_pool.shape[1])


def _i32(t, name: str, device):
    torch = _torch()
    if t.dtype != torch.int32 or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor on {device}")
    return t.data_ptr()


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def make_workspace(p: PaPlan, total_rows: int, head_dim: int, device):
    """(acc, max, sum) for the plan; a batch plan (ragged splits) also gets the
    split index, and its rows are one KV unit's (total_rows is not used)."""
    torch = _torch()
    if p.selection == PA_SELECTION["batch"]:
        total_rows = p.rows_per_kv_unit
    acc = torch.empty((p.num_splits, total_rows, head_dim), dtype=torch.float32, device=device)
    mx = torch.empty((p.num_splits, total_rows), dtype=torch.float32, device=device)
    sm = torch.empty((p.num_splits, total_rows), dtype=torch.float32, device=device)
    if p.selection == PA_SELECTION["batch"]:
        idx = torch.empty(p.num_kv_units + 1, dtype=torch.int32, device=device)
        return acc, mx, sm, idx
    return acc, mx, sm


def _ws(acc, mx, sm, index=None) -> PaWorkspace:
    torch = _torch()
    for t in (acc, mx, sm):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("workspace buffers must be contiguous float32")
    if index is not None and (index.dtype != torch.int32 or not index.is_contiguous()):
        raise ValueError("the split index must be a contiguous int32 tensor")
    return PaWorkspace(acc.data_ptr(), mx.data_ptr(), sm.data_ptr(),
                       acc.numel() * 4, min(mx.numel(), sm.numel()) * 4,
                       None if index is None else index.data_ptr(),
                       0 if index is None else index.numel() * 4)


def paged_attn_verify_e4m3(q, k_pool, v_pool, block_table, row_lens, max_tokens: int,
                           sm_scale, k_scale, p: PaPlan, ws) -> None:
    """Dense verify of one request into the FP32 split workspace ws = (acc, max, sum)."""
    torch = _torch()
    if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 3:
        raise ValueError("q must be a contiguous float16 tensor [q_rows][heads][head_dim]")
    dev = q.device
    pool = _pool(k_pool, v_pool, dev)
    qr, H, D = q.shape
    if k_pool.shape[3] != D:
        raise ValueError("head_dim of q and the pool differ")
    rc = lib().paged_attn_verify_e4m3(
        q.data_ptr(), ctypes.byref(pool), _i32(block_table, "block_table", dev),
        block_table.numel(), _i32(row_lens, "row_lens", dev), int(max_tokens), qr, H,
        k_pool.shape[2], D, _scale(sm_scale, "sm_scale"), _scale(k_scale, "k_scale"),
        ctypes.byref(p), ctypes.byref(_ws(*ws)), _stream(dev))
    _check(rc, "paged_attn_verify_e4m3")


NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024


def paged_attn_verify_noalloc_e4m3(q, k_pool, v_pool, block_table, row_lens, max_tokens: int,
                                   sm_scale, k_scale, v_scale, p: PaPlan, out) -> None:
    """Dense verify + combine of one request into out (float16, contiguous
    [q_rows][heads][head_dim]) with the split partials in the library's fixed
    per-device scratch: no workspace, nothing allocated."""
    torch = _torch()
    if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 3:
        raise ValueError("q must be a contiguous float16 tensor [q_rows][heads][head_dim]")
    dev = q.device
    pool = _pool(k_pool, v_pool, dev)
    qr, H, D = q.shape
    if k_pool.shape[3] != D:
        raise ValueError("head_dim of q and the pool differ")
    if out.dtype != torch.float16 or not out.is_contiguous() or out.numel() < qr * H * D \
            or out.device != dev:
        raise ValueError("out must be a contiguous float16 tensor of q_rows*heads*head_dim "
                         "elements on the query's device")
    rc = lib().paged_attn_verify_noalloc_e4m3(
        q.data_ptr(), ctypes.byref(pool), _i32(block_table, "block_table", dev),
        block_table.numel(), _i32(row_lens, "row_lens", dev), int(max_tokens), qr, H,
        k_pool.shape[2], D, _scale(sm_scale, "sm_scale"), _scale(k_scale, "k_scale"),
        _scale(v_scale, "v_scale"), ctypes.byref(p), out.data_ptr(), _stream(dev))
    _check(rc, "paged_attn_verify_noalloc_e4m3")


def paged_attn_verify_batch_e4m3(q, k_pool, v_pool, block_table, row_lens, sm_scale, k_scale,
                                 p: PaPlan, ws) -> None:
    """Dense verify of a batch of independent requests into the FP32 split workspace."""
    torch = _torch()
    if q.dtype != torch.float16 or not q.is_contiguous() or q.dim() != 4:
        raise ValueError("q must be a contiguous float16 tensor [batch][q_rows][heads][head_dim]")
    dev = q.device
    pool = _pool(k_pool, v_pool, dev)
    B, qr, H, D = q.shape
    if k_pool.shape[3] != D:
        raise ValueError("head_dim of q and the pool differ")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch][max_blocks]")
    if tuple(row_lens.shape) != (B, qr):
        raise ValueError("row_lens must be [batch][q_rows]")
    Hkv = k_pool.shape[2]
    rc = lib().paged_attn_verify_batch_e4m3(
        q.data_ptr(), ctypes.byref(pool), _i32(block_table, "block_table", dev),
        block_table.shape[1], _i32(row_lens, "row_lens", dev), B, qr, H, Hkv, D,
        _scale(sm_scale, "sm_scale"), _scale(k_scale, "k_scale"), ctypes.byref(p),
        ctypes.byref(_ws(*ws)), _stream(dev))
    _check(rc, "paged_attn_verify_batch_e4m3")


def paged_attn_cache_write_e4m3(k, v, slot_mapping, k_pool, v_pool, k_scale, v_scale) -> None:
    """Write FP16 K/V tokens (contiguous [num_tokens][kv_heads][head_dim]) into the
    E4M3 pools ([pages][page_size][kv_heads][head_dim] uint8 views) by slot
    (int64 [num_tokens]; < 0 skipped)."""
    torch = _torch()
    for t in (k, v):
        if t.dtype != torch.float16 or not t.is_contiguous() or t.dim() != 3:
            raise ValueError("k and v must be contiguous float16 [num_tokens][kv_heads][head_dim]")
    if k.shape != v.shape:
        raise ValueError("k and v shapes differ")
    dev = k.device
    T, Hkv, D = k.shape
    if slot_mapping.dtype != torch.int64 or slot_mapping.device != dev or \
            not slot_mapping.is_contiguous() or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be a contiguous int64 tensor of num_tokens on k's device")
    if k_pool.shape[2] != Hkv or k_pool.shape[3] != D:
        raise ValueError("pool heads or head_dim differ from k")
    pool = _pool(k_pool, v_pool, dev)
    rc = lib().paged_attn_cache_write_e4m3(k.data_ptr(), v.data_ptr(), T, Hkv, D,
                                           slot_mapping.data_ptr(), ctypes.byref(pool),
                                           _scale(k_scale, "k_scale"),
                                           _scale(v_scale, "v_scale"), _stream(dev))
    _check(rc, "paged_attn_cache_write_e4m3")


def paged_attn_combine_batch_fp32(ws, p: PaPlan, batch: int, q_rows: int, num_heads: int,
                                  num_kv_heads: int, head_dim: int, out_scale, out) -> None:
    """FP32 combine of a batch's ragged partials (ws = (acc, max, sum, index) as
    paged_attn_verify_batch_e4m3 wrote them with plan p) into out (float16,
    [batch][q_rows][heads][head_dim] elements)."""
    torch = _torch()
    if len(ws) != 4:
        raise ValueError("a batch workspace is (acc, max, sum, index)")
    if out.dtype != torch.float16 or not out.is_contiguous() or \
            out.numel() < batch * q_rows * num_heads * head_dim or out.device != ws[0].device:
        raise ValueError("out must be a contiguous float16 tensor of batch*q_rows*heads*head_dim "
                         "elements on the workspace's device")
    rc = lib().paged_attn_combine_batch_fp32(ctypes.byref(_ws(*ws)), ctypes.byref(p), int(batch),
                                             int(q_rows), int(num_heads), int(num_kv_heads),
                                             int(head_dim), _scale(out_scale, "out_scale"),
                                             out.data_ptr(), _stream(out.device))
    _check(rc, "paged_attn_combine_batch_fp32")


def paged_attn_combine_batch_fp32_lse(ws, p: PaPlan, batch: int, q_rows: int,
                                      num_heads: int, num_kv_heads: int, head_dim: int,
                                      out_scale, out=None, out32=None, lse=None) -> None:
    """The batch combine writing any of: out (float16), out32 (float32), both
    [batch][q_rows][heads][head_dim] elements, and lse (float32,
    [batch][q_rows][heads]): the base-2 LSE of each row, for a merge across ranks."""
    torch = _torch()
    if len(ws) != 4:
        raise ValueError("a batch workspace is (acc, max, sum, index)")
    if out is None and out32 is None and lse is None:
        raise ValueError("give at least one of out, out32, lse")
    rows = batch * q_rows * num_heads
    dev = ws[0].device
    for t, dt, n in ((out, torch.float16, rows * head_dim), (out32, torch.float32, rows * head_dim),
                     (lse, torch.float32, rows)):
        if t is not None and (t.dtype != dt or not t.is_contiguous() or t.numel() < n
                              or t.device != dev):
            raise ValueError(f"outputs must be contiguous {dt} tensors of {n} elements on {dev}")
    ptr = lambda t: None if t is None else t.data_ptr()
    rc = lib().paged_attn_combine_batch_fp32_lse(ctypes.byref(_ws(*ws)), ctypes.byref(p),
                                                 int(batch), int(q_rows), int(num_heads),
                                                 int(num_kv_heads), int(head_dim),
                                                 _scale(out_scale, "out_scale"), ptr(out),
                                                 ptr(out32), ptr(lse), _stream(dev))
    _check(rc, "paged_attn_combine_batch_fp32_lse")


def paged_attn_combine_fp32(ws, num_splits: int, num_rows: int, head_dim: int, out_scale,
                            out) -> None:
    """FP32 combine of split partials into out (float16, [num_rows][head_dim] elements)."""
    torch = _torch()
    acc, mx, sm = ws[:3]
    if out.dtype != torch.float16 or not out.is_contiguous() or out.numel() < num_rows * head_dim:
        raise ValueError("out must be a contiguous float16 tensor of num_rows*head_dim elements")
    for t in (acc, mx, sm):
        if t.device != out.device or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("workspace must be contiguous float32 on the output's device")
    if acc.numel() < num_splits * num_rows * head_dim or min(mx.numel(), sm.numel()) < num_splits * num_rows:
        raise ValueError("workspace smaller than num_splits x num_rows")
    rc = lib().paged_attn_combine_fp32(acc.data_ptr(), mx.data_ptr(), sm.data_ptr(),
                                       int(num_splits), int(num_rows), int(head_dim),
                                       _scale(out_scale, "out_scale"),
                                       out.data_ptr(), _stream(out.device))
    _check(rc, "paged_attn_combine_fp32")


def paged_attn_combine_fp32_lse(ws, num_splits: int, num_rows: int, head_dim: int, out_scale,
                                out=None, out32=None, lse=None) -> None:
    """FP32 combine writing any of: out (float16), out32 (float32), both
    [num_rows][head_dim] elements, and lse (float32, num_rows): the base-2 LSE of
    each row, for a merge across ranks."""
    torch = _torch()
    acc, mx, sm = ws[:3]
    if out is None and out32 is None and lse is None:
        raise ValueError("give at least one of out, out32, lse")
    dev = acc.device
    for t, dt, n in ((out, torch.float16, num_rows * head_dim),
                     (out32, torch.float32, num_rows * head_dim), (lse, torch.float32, num_rows)):
        if t is not None and (t.dtype != dt or not t.is_contiguous() or t.numel() < n
                              or t.device != dev):
            raise ValueError(f"outputs must be contiguous {dt} tensors of {n} elements on {dev}")
    for t in (acc, mx, sm):
        if t.device != dev or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("workspace must be contiguous float32 on one device")
    if acc.numel() < num_splits * num_rows * head_dim or min(mx.numel(), sm.numel()) < num_splits * num_rows:
        raise ValueError("workspace smaller than num_splits x num_rows")
    ptr = lambda t: None if t is None else t.data_ptr()
    rc = lib().paged_attn_combine_fp32_lse(acc.data_ptr(), mx.data_ptr(), sm.data_ptr(),
                                           int(num_splits), int(num_rows), int(head_dim),
                                           _scale(out_scale, "out_scale"), ptr(out),
                                           ptr(out32), ptr(lse), _stream(dev))
    _check(rc, "paged_attn_combine_fp32_lse")


def _sparse_args(q, k_pool, v_pool, block_table, sel, row_lens, name):
    torch = _torch()
    if q.dtype != torch.bfloat16 or not q.is_contiguous() or q.dim() != 4:
        raise ValueError("q must be a contiguous bfloat16 tensor [batch][q_rows][heads][head_dim]")
    dev = q.device
    pool = _pool(k_pool, v_pool, dev)
    B, qr, H, D = q.shape
    if k_pool.shape[3] != D:
        raise ValueError("head_dim of q and the pool differ")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [batch][max_blocks]")
    Hkv = k_pool.shape[2]
    if sel.dim() != 3 or tuple(sel.shape[:2]) != (B, Hkv):
        raise ValueError(f"{name} must be [batch][kv_heads][n]")
    if tuple(row_lens.shape) != (B, qr):
        raise ValueError("row_lens must be [batch][q_rows]")
    return (q.data_ptr(), ctypes.byref(pool), _i32(block_table, "block_table", dev),
            block_table.shape[1], _i32(sel, name, dev), sel.shape[2],
            _i32(row_lens, "row_lens", dev), B, qr, H, Hkv, D), dev


def qsa_sparse_verify_e4m3(q, k_pool, v_pool, block_table, sel_blocks, row_lens, sm_scale,
                           k_scale, p: PaPlan, ws) -> None:
    """Sparse verify of a batch over selected blocks into the FP32 split workspace."""
    args, dev = _sparse_args(q, k_pool, v_pool, block_table, sel_blocks, row_lens,
                             "sel_blocks")
    rc = lib().qsa_sparse_verify_e4m3(
        *args, _scale(sm_scale, "sm_scale"), _scale(k_scale, "k_scale"),
        ctypes.byref(p), ctypes.byref(_ws(*ws)), _stream(dev))
    _check(rc, "qsa_sparse_verify_e4m3")


def qsa_sparse_verify_tokens_e4m3(q, k_pool, v_pool, block_table, sel_tokens, row_lens,
                                  sm_scale, k_scale, p: PaPlan, ws) -> None:
    """Sparse verify of a batch over selected token ids (-1 = empty) into the
    FP32 split workspace."""
    args, dev = _sparse_args(q, k_pool, v_pool, block_table, sel_tokens, row_lens,
                             "sel_tokens")
    rc = lib().qsa_sparse_verify_tokens_e4m3(
        *args, _scale(sm_scale, "sm_scale"), _scale(k_scale, "k_scale"),
        ctypes.byref(p), ctypes.byref(_ws(*ws)), _stream(dev))
    _check(rc, "qsa_sparse_verify_tokens_e4m3")


# ---------------------------------------------------------------------------
# Conveniences: verify + combine
# ---------------------------------------------------------------------------


def verify(q, k_pool, v_pool, block_table, row_lens, max_tokens: int, *, sm_scale, k_scale,
           v_scale, splits: int = 0, kernel: str = "auto", p: Optional[PaPlan] = None,
           ws: Optional[Tuple] = None, out=None):
    """Dense verify of one request; returns FP16 [q_rows][heads][head_dim]."""
    torch = _torch()
    qr, H, D = q.shape
    Hkv = k_pool.shape[2]
    if p is None:
        p = plan(max_tokens, qr * (H // Hkv), Hkv, D, k_pool.shape[1], splits=splits,
                 kernel=kernel)
    if ws is None:
        ws = make_workspace(p, qr * H, D, q.device)
    if out is None:
        out = torch.empty((qr, H, D), dtype=torch.float16, device=q.device)
    paged_attn_verify_e4m3(q, k_pool, v_pool, block_table, row_lens, max_tokens, sm_scale,
                           k_scale, p, ws)
    paged_attn_combine_fp32(ws, p.num_splits, qr * H, D, v_scale, out)
    return out


def verify_batch(q, k_pool, v_pool, block_table, row_lens, *, sm_scale, k_scale, v_scale,
                 splits: int = 0, kernel: str = "auto", p: Optional[PaPlan] = None,
                 ws: Optional[Tuple] = None, out=None):
    """Dense verify of a batch of requests; returns FP16 [batch][q_rows][heads][head_dim]."""
    torch = _torch()
    B, qr, H, D = q.shape
    Hkv = k_pool.shape[2]
    cap = block_table.shape[1] * k_pool.shape[1]
    if p is None:
        p = plan(cap, qr * (H // Hkv), B * Hkv, D, k_pool.shape[1], "batch", splits=splits,
                 kernel=kernel)
    if ws is None:
        ws = make_workspace(p, B * qr * H, D, q.device)
    if out is None:
        out = torch.empty((B, qr, H, D), dtype=torch.float16, device=q.device)
    paged_attn_verify_batch_e4m3(q, k_pool, v_pool, block_table, row_lens, sm_scale, k_scale,
                                 p, ws)
    paged_attn_combine_batch_fp32(ws, p, B, qr, H, Hkv, D, v_scale, out)
    return out


def qsa_verify(q, k_pool, v_pool, block_table, sel_blocks, row_lens, *, sm_scale, k_scale,
               v_scale, splits: int = 0, kernel: str = "auto", p: Optional[PaPlan] = None,
               ws: Optional[Tuple] = None, out=None):
    """Sparse verify of a batch; returns FP16 [batch][q_rows][heads][head_dim]."""
    torch = _torch()
    B, qr, H, D = q.shape
    Hkv = k_pool.shape[2]
    page = k_pool.shape[1]
    if p is None:
        p = plan(sel_blocks.shape[2] * page, qr * (H // Hkv), B * Hkv, D, page, "blocks",
                 splits=splits, kernel=kernel)
    if ws is None:
        ws = make_workspace(p, B * qr * H, D, q.device)
    if out is None:
        out = torch.empty((B, qr, H, D), dtype=torch.float16, device=q.device)
    qsa_sparse_verify_e4m3(q, k_pool, v_pool, block_table, sel_blocks, row_lens, sm_scale,
                           k_scale, p, ws)
    paged_attn_combine_fp32(ws, p.num_splits, B * qr * H, D, v_scale, out)
    return out


def qsa_verify_tokens(q, k_pool, v_pool, block_table, sel_tokens, row_lens, *, sm_scale,
                      k_scale, v_scale, splits: int = 0, kernel: str = "auto",
                      p: Optional[PaPlan] = None, ws: Optional[Tuple] = None, out=None):
    """Sparse verify of a batch over selected token ids; returns FP16
    [batch][q_rows][heads][head_dim]."""
    torch = _torch()
    B, qr, H, D = q.shape
    Hkv = k_pool.shape[2]
    if p is None:
        p = plan(sel_tokens.shape[2], qr * (H // Hkv), B * Hkv, D, k_pool.shape[1], "tokens",
                 splits=splits, kernel=kernel)
    if ws is None:
        ws = make_workspace(p, B * qr * H, D, q.device)
    if out is None:
        out = torch.empty((B, qr, H, D), dtype=torch.float16, device=q.device)
    qsa_sparse_verify_tokens_e4m3(q, k_pool, v_pool, block_table, sel_tokens, row_lens,
                                  sm_scale, k_scale, p, ws)
    paged_attn_combine_fp32(ws, p.num_splits, B * qr * H, D, v_scale, out)
    return out
