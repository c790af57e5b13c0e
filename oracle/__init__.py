"""FP64 CPU oracle for multi-row verify attention over a paged E4M3 KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this package; the product library never
does, and this package imports nothing from the product.  The arithmetic
lives in ``oracle.c`` (plain C, FP64); this module only marshals numpy arrays
through ctypes.  Build it with ``oracle.build.build()``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_i32, _i64, _f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
_p = ctypes.c_void_p


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Oracle:
    """ctypes view of one built liboracle (the normal one or a planted-mistake build)."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise FileNotFoundError(f"{path} missing: run oracle.build.build() first")
        self.path = path
        lib = ctypes.CDLL(path)
        lib.orc_e4m3_table.argtypes = [_p]
        lib.orc_e4m3_table.restype = None
        lib.orc_e4m3_encode.argtypes = [_f64]
        lib.orc_e4m3_encode.restype = ctypes.c_uint8
        lib.orc_e4m3_encode_array.argtypes = [_p, _i64, _p]
        lib.orc_e4m3_encode_array.restype = None
        lib.orc_cache_write.argtypes = [_p, _p, _i64, _i32, _i32, _p, _p, _p, _i64, _i64, _i64,
                                        _i32, _i32, ctypes.c_float, ctypes.c_float]
        lib.orc_cache_write.restype = ctypes.c_int
        lib.orc_fp16_value.argtypes = [ctypes.c_uint16]
        lib.orc_fp16_value.restype = _f64
        lib.orc_bf16_value.argtypes = [ctypes.c_uint16]
        lib.orc_bf16_value.restype = _f64
        pool = [_p, _p, _p, _i64, _i64, _i64, _i32, _i32]
        lib.orc_verify_dense.argtypes = pool + [_p, _i32, _p, _i32, _i32, _i32, _i32, _i32,
                                                _f64, _f64, _f64, _i32, _p]
        lib.orc_verify_dense.restype = ctypes.c_int
        lib.orc_verify_dense_split.argtypes = pool + [_p, _i32, _p, _i32, _i32, _i32, _i32,
                                                      _i32, _f64, _f64, _i32, _i32, _i32,
                                                      _p, _p, _p]
        lib.orc_verify_dense_split.restype = ctypes.c_int
        lib.orc_qsa_verify.argtypes = pool + [_p, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                              _i32, _f64, _f64, _f64, _i32, _p]
        lib.orc_qsa_verify.restype = ctypes.c_int
        lib.orc_qsa_split.argtypes = pool + [_p, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                             _i32, _f64, _f64, _i32, _i32, _i32, _p, _p, _p]
        lib.orc_qsa_split.restype = ctypes.c_int
        lib.orc_qsa_tokens_verify.argtypes = pool + [_p, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                              _i32, _f64, _f64, _f64, _i32, _p]
        lib.orc_qsa_tokens_verify.restype = ctypes.c_int
        lib.orc_qsa_tokens_split.argtypes = pool + [_p, _i32, _p, _i32, _p, _i32, _i32, _i32, _i32,
                                             _i32, _f64, _f64, _i32, _i32, _i32, _p, _p, _p]
        lib.orc_qsa_tokens_split.restype = ctypes.c_int
        lib.orc_combine.argtypes = [_p, _p, _p, _i32, _i32, _i32, _f64, _p]
        lib.orc_combine.restype = ctypes.c_int
        lib.orc_combine_f32.argtypes = [_p, _p, _p, _i32, _i32, _i32, _f64, _p]
        lib.orc_combine_f32.restype = ctypes.c_int
        lib.orc_combine_lse.argtypes = [_p, _p, _p, _i32, _i32, _i32, _f64, _p, _p]
        lib.orc_combine_lse.restype = ctypes.c_int
        lib.orc_combine_lse_f32.argtypes = [_p, _p, _p, _i32, _i32, _i32, _f64, _p, _p]
        lib.orc_combine_lse_f32.restype = ctypes.c_int
        self.lib = lib

    # -- number formats ------------------------------------------------------
    def e4m3_table(self) -> np.ndarray:
        t = np.empty(256, np.float64)
        self.lib.orc_e4m3_table(_ptr(t))
        return t

    def cache_write(self, k_bits, v_bits, slot_mapping, k_pool, v_pool, k_scale, v_scale):
        """Write FP16 K/V tokens ([T][Hkv][D] bit patterns) into copies of the
        E4M3 pools ([pages][page_size][Hkv][D], contiguous) by slot; returns
        the new (k_pool, v_pool)."""
        k_bits = np.ascontiguousarray(k_bits, np.uint16)
        v_bits = np.ascontiguousarray(v_bits, np.uint16)
        slots = np.ascontiguousarray(slot_mapping, np.int64)
        kp = np.array(k_pool, np.uint8, copy=True, order="C")
        vp = np.array(v_pool, np.uint8, copy=True, order="C")
        T, Hkv, D = k_bits.shape
        P, ps = kp.shape[0], kp.shape[1]
        rc = self.lib.orc_cache_write(_ptr(k_bits), _ptr(v_bits), T, Hkv, D, _ptr(slots),
                                      _ptr(kp), _ptr(vp), ps * Hkv * D, Hkv * D, D, P, ps,
                                      float(k_scale), float(v_scale))
        if rc != 0:
            raise ValueError("orc_cache_write: slot out of range")
        return kp, vp

    def e4m3_encode(self, x) -> np.ndarray:
        x = np.ascontiguousarray(np.asarray(x, np.float64).ravel())
        out = np.empty(x.size, np.uint8)
        self.lib.orc_e4m3_encode_array(_ptr(x), x.size, _ptr(out))
        return out

    def fp16_value(self, bits: int) -> float:
        return self.lib.orc_fp16_value(int(bits))

    def bf16_value(self, bits: int) -> float:
        return self.lib.orc_bf16_value(int(bits))

    # -- attention -------------------------------------------------------------
    @staticmethod
    def _pool_args(k_pool: np.ndarray, v_pool: np.ndarray, strides=None):
        """Pool pointers and byte strides; default: contiguous [P][page][Hkv][D]."""
        assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
        assert k_pool.shape == v_pool.shape
        P, page = k_pool.shape[0], k_pool.shape[1]
        if strides is None:
            strides = (k_pool.strides[0], k_pool.strides[1], k_pool.strides[2])
            assert k_pool.strides == v_pool.strides
        return [_ptr(k_pool), _ptr(v_pool), strides[0], strides[1], strides[2], P, page]

    def verify_dense(self, q_bits, k_pool, v_pool, block_table, row_lens, max_tokens,
                     num_kv_heads, sm_scale, k_scale, v_scale, nthreads=1,
                     strides=None, page_size=None, num_pages=None) -> np.ndarray:
        q_bits = np.ascontiguousarray(q_bits, np.uint16)
        bt = np.ascontiguousarray(block_table, np.int32)
        rl = np.ascontiguousarray(row_lens, np.int32)
        qr, H, D = q_bits.shape
        out = np.empty((qr, H, D), np.float64)
        pa = self._pool_args(k_pool, v_pool, strides)
        if page_size is not None:
            pa[6] = page_size
        if num_pages is not None:
            pa[5] = num_pages
        rc = self.lib.orc_verify_dense(_ptr(q_bits), *pa, _ptr(bt), bt.size, _ptr(rl),
                                       int(max_tokens), qr, H, int(num_kv_heads), D,
                                       float(sm_scale), float(k_scale), float(v_scale),
                                       int(nthreads), _ptr(out))
        if rc != 0:
            raise ValueError(f"orc_verify_dense precondition failed ({rc})")
        return out

    def verify_dense_split(self, q_bits, k_pool, v_pool, block_table, row_lens, max_tokens,
                           num_kv_heads, sm_scale, k_scale, num_splits, tokens_per_split,
                           nthreads=1, strides=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        q_bits = np.ascontiguousarray(q_bits, np.uint16)
        bt = np.ascontiguousarray(block_table, np.int32)
        rl = np.ascontiguousarray(row_lens, np.int32)
        qr, H, D = q_bits.shape
        R = qr * H
        acc = np.empty((num_splits, R, D), np.float64)
        mx = np.empty((num_splits, R), np.float64)
        sm = np.empty((num_splits, R), np.float64)
        rc = self.lib.orc_verify_dense_split(
            _ptr(q_bits), *self._pool_args(k_pool, v_pool, strides), _ptr(bt), bt.size,
            _ptr(rl), int(max_tokens), qr, H, int(num_kv_heads), D, float(sm_scale),
            float(k_scale), int(num_splits), int(tokens_per_split), int(nthreads),
            _ptr(acc), _ptr(mx), _ptr(sm))
        if rc != 0:
            raise ValueError(f"orc_verify_dense_split precondition failed ({rc})")
        return acc, mx, sm

    def qsa_verify(self, q_bits, k_pool, v_pool, block_table, sel_blocks, row_lens,
                   sm_scale, k_scale, v_scale, nthreads=1, strides=None) -> np.ndarray:
        q_bits = np.ascontiguousarray(q_bits, np.uint16)
        bt = np.ascontiguousarray(block_table, np.int32)
        sel = np.ascontiguousarray(sel_blocks, np.int32)
        rl = np.ascontiguousarray(row_lens, np.int32)
        B, qr, H, D = q_bits.shape
        Hkv, topk = sel.shape[1], sel.shape[2]
        out = np.empty((B, qr, H, D), np.float64)
        rc = self.lib.orc_qsa_verify(
            _ptr(q_bits), *self._pool_args(k_pool, v_pool, strides), _ptr(bt), bt.shape[1],
            _ptr(sel), topk, _ptr(rl), B, qr, H, Hkv, D, float(sm_scale), float(k_scale),
            float(v_scale), int(nthreads), _ptr(out))
        if rc != 0:
            raise ValueError(f"orc_qsa_verify precondition failed ({rc})")
        return out

    def qsa_split(self, q_bits, k_pool, v_pool, block_table, sel_blocks, row_lens,
                  sm_scale, k_scale, num_splits, tokens_per_split, nthreads=1,
                  strides=None):
        q_bits = np.ascontiguousarray(q_bits, np.uint16)
        bt = np.ascontiguousarray(block_table, np.int32)
        sel = np.ascontiguousarray(sel_blocks, np.int32)
        rl = np.ascontiguousarray(row_lens, np.int32)
        B, qr, H, D = q_bits.shape
        Hkv, topk = sel.shape[1], sel.shape[2]
        R = B * qr * H
        acc = np.empty((num_splits, R, D), np.float64)
        mx = np.empty((num_splits, R), np.float64)
        sm = np.empty((num_splits, R), np.float64)
        rc = self.lib.orc_qsa_split(
            _ptr(q_bits), *self._pool_args(k_pool, v_pool, strides), _ptr(bt), bt.shape[1],
            _ptr(sel), topk, _ptr(rl), B, qr, H, Hkv, D, float(sm_scale), float(k_scale),
            int(num_splits), int(tokens_per_split), int(nthreads), _ptr(acc), _ptr(mx),
            _ptr(sm))
        if rc != 0:
            raise ValueError(f"orc_qsa_split precondition failed ({rc})")
        return acc, mx, sm

    def qsa_tokens_verify(self, q_bits, k_pool, v_pool, block_table, sel_tokens, row_lens,
                          sm_scale, k_scale, v_scale, nthreads=1, strides=None) -> np.ndarray:
        q_bits = np.ascontiguousarray(q_bits, np.uint16)
        bt = np.ascontiguousarray(block_table, np.int32)
        sel = np.ascontiguousarray(sel_tokens, np.int32)
        rl = np.ascontiguousarray(row_lens, np.int32)
        B, qr, H, D = q_bits.shape
        Hkv, topk = sel.shape[1], sel.shape[2]
        out = np.empty((B, qr, H, D), np.float64)
        rc = self.lib.orc_qsa_tokens_verify(
            _ptr(q_bits), *self._pool_args(k_pool, v_pool, strides), _ptr(bt), bt.shape[1],
            _ptr(sel), topk, _ptr(rl), B, qr, H, Hkv, D, float(sm_scale), float(k_scale),
            float(v_scale), int(nthreads), _ptr(out))
        if rc != 0:
            raise ValueError(f"orc_qsa_tokens_verify precondition failed ({rc})")
        return out

    def qsa_tokens_split(self, q_bits, k_pool, v_pool, block_table, sel_tokens, row_lens,
                         sm_scale, k_scale, num_splits, tokens_per_split, nthreads=1,
                         strides=None):
        q_bits = np.ascontiguousarray(q_bits, np.uint16)
        bt = np.ascontiguousarray(block_table, np.int32)
        sel = np.ascontiguousarray(sel_tokens, np.int32)
        rl = np.ascontiguousarray(row_lens, np.int32)
        B, qr, H, D = q_bits.shape
        Hkv, topk = sel.shape[1], sel.shape[2]
        R = B * qr * H
        acc = np.empty((num_splits, R, D), np.float64)
        mx = np.empty((num_splits, R), np.float64)
        sm = np.empty((num_splits, R), np.float64)
        rc = self.lib.orc_qsa_tokens_split(
            _ptr(q_bits), *self._pool_args(k_pool, v_pool, strides), _ptr(bt), bt.shape[1],
            _ptr(sel), topk, _ptr(rl), B, qr, H, Hkv, D, float(sm_scale), float(k_scale),
            int(num_splits), int(tokens_per_split), int(nthreads), _ptr(acc), _ptr(mx),
            _ptr(sm))
        if rc != 0:
            raise ValueError(f"orc_qsa_tokens_split precondition failed ({rc})")
        return acc, mx, sm

    def combine(self, acc, mx, sm, v_scale, with_lse: bool = False):
        """Merge split partials (FP64 or FP32 arrays) into FP64 rows; with
        with_lse, also the base-2 LSE of each row: returns (out, lse)."""
        S, R, D = acc.shape
        out = np.empty((R, D), np.float64)
        lse = np.empty(R, np.float64)
        f32 = acc.dtype == np.float32
        dt = np.float32 if f32 else np.float64
        acc = np.ascontiguousarray(acc, dt)
        mx = np.ascontiguousarray(mx, dt)
        sm = np.ascontiguousarray(sm, dt)
        if with_lse:
            fn = self.lib.orc_combine_lse_f32 if f32 else self.lib.orc_combine_lse
            rc = fn(_ptr(acc), _ptr(mx), _ptr(sm), S, R, D, float(v_scale), _ptr(out), _ptr(lse))
        else:
            fn = self.lib.orc_combine_f32 if f32 else self.lib.orc_combine
            rc = fn(_ptr(acc), _ptr(mx), _ptr(sm), S, R, D, float(v_scale), _ptr(out))
        if rc != 0:
            raise ValueError("orc_combine failed")
        return (out, lse) if with_lse else out

    # -- conveniences over the seeded workloads --------------------------------
    def dense_workload(self, w, nthreads=1) -> np.ndarray:
        return self.verify_dense(w.q_bits, w.k_pool, w.v_pool, w.block_table, w.row_lens,
                                 w.max_tokens, w.num_kv_heads, w.sm_scale, w.k_scale,
                                 w.v_scale, nthreads=nthreads)

    def qsa_workload(self, w, nthreads=1) -> np.ndarray:
        return self.qsa_verify(w.q_bits, w.k_pool, w.v_pool, w.block_table, w.sel_blocks,
                               w.row_lens, w.sm_scale, w.k_scale, w.v_scale,
                               nthreads=nthreads)

    def qsa_tokens_workload(self, w, nthreads=1) -> np.ndarray:
        return self.qsa_tokens_verify(w.q_bits, w.k_pool, w.v_pool, w.block_table,
                                      w.sel_tokens, w.row_lens, w.sm_scale, w.k_scale,
                                      w.v_scale, nthreads=nthreads)


_DEFAULT: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from oracle.c with no planted mistake."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(LIB_PATH)
    return _DEFAULT
