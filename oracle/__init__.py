"""CPU oracle for MoE expert-parallel layout / dispatch / combine.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.
It is a thin numpy front end over ``ep_oracle.c`` (plain C, gcc, no HIP),
which holds every step of the arithmetic; see that file's header for the
passages each function follows and the readings taken where the pages are
silent.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)

_LIBS = {}


def lib(path: str = None):
    """Load the oracle library (default: liboracle_ep.so, compiled if missing)."""
    if path is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    if path not in _LIBS:
        L = ctypes.CDLL(path)
        L.oracle_layout.argtypes = [_i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, _i32p, _i32p, _i32p, _i32p, _i32p]
        L.oracle_layout.restype = ctypes.c_int
        L.oracle_dispatch.argtypes = [_u8p, ctypes.c_int64, _u8p, ctypes.c_int64, _f32p, _i32p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                      _u8p, _u8p, _f32p]
        L.oracle_dispatch.restype = ctypes.c_int
        L.oracle_combine.argtypes = [_u16p, ctypes.c_int32, _f32p, _u16p, _i32p, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int64, _u16p]
        L.oracle_combine.restype = ctypes.c_int
        L.oracle_combine_f32.argtypes = [_f32p, ctypes.c_int32, _f32p, _f32p, _i32p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int64, _f32p]
        L.oracle_combine_f32.restype = ctypes.c_int
        L.oracle_dispatch_compact.argtypes = [_u8p, ctypes.c_int64, _u8p, ctypes.c_int64, _i32p, _f32p,
                                              _i32p, _i32p, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, _u8p, _u8p, _i32p, _f32p]
        L.oracle_dispatch_compact.restype = ctypes.c_int
        L.oracle_combine_compact.argtypes = [_u16p, ctypes.c_int32, _u16p, _i32p, _i32p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, _u16p]
        L.oracle_combine_compact.restype = ctypes.c_int
        L.oracle_combine_compact_f32.argtypes = [_f32p, ctypes.c_int32, _f32p, _i32p, _i32p,
                                                 ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                 _f32p]
        L.oracle_combine_compact_f32.restype = ctypes.c_int
        L.oracle_zero_padding.argtypes = [_u8p, ctypes.c_int64, _u8p, ctypes.c_int64, _f32p, _i32p,
                                          _i32p, ctypes.c_int32, ctypes.c_int64]
        L.oracle_zero_padding.restype = ctypes.c_int
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        _LIBS[path] = L
    return _LIBS[path]


def _ptr(a, typ):
    if a is None:
        return ctypes.cast(None, typ)
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(typ)


def layout(topk_idx: np.ndarray, num_experts: int, expert_alignment: int, _lib=None):
    """Counts, aligned exclusive offsets, slots and receive metadata.

    Returns a dict with ``counts`` int32[E], ``offsets`` int32[E+1],
    ``dst_slot`` int32[T,K], ``recv_src_metadata`` int32[num_recv,K+2]
    and ``num_recv`` (int).
    """
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = idx.shape
    E, A = int(num_experts), int(expert_alignment)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    dst = np.zeros((T, K), np.int32)
    meta = np.zeros((max(T, 1), K + 2), np.int32)
    nrecv = np.zeros(1, np.int32)
    rc = lib(_lib).oracle_layout(_ptr(idx, _i32p), T, K, E, A, _ptr(counts, _i32p),
                             _ptr(offsets, _i32p), _ptr(dst, _i32p), _ptr(meta, _i32p),
                             _ptr(nrecv, _i32p))
    if rc != 0:
        raise ValueError("oracle_layout rejected its arguments")
    n = int(nrecv[0])
    return {"counts": counts, "offsets": offsets, "dst_slot": dst,
            "recv_src_metadata": meta[:n].copy(), "num_recv": n}


def _byte_rows(a: np.ndarray, rows: int) -> np.ndarray:
    """a as contiguous uint8 [rows, bytes per row]; the row length comes from
    a's shape, so an array with zero rows keeps its width."""
    a = np.ascontiguousarray(a)
    width = int(np.prod(a.shape[1:], dtype=np.int64)) * a.itemsize if a.ndim > 1 else a.itemsize
    return a.view(np.uint8).reshape(rows, width)


def dispatch(x_bytes: np.ndarray, dst_slot: np.ndarray, capacity_rows: int,
             x_scales: np.ndarray = None, topk_weights: np.ndarray = None,
             expand_x: np.ndarray = None, expand_scales: np.ndarray = None,
             expand_weights: np.ndarray = None, _lib=None):
    """Permute-copy token rows (any dtype, moved as bytes) to the expand buffer.

    ``x_bytes`` is [T, row_bytes] uint8 (a view of bf16 or fp8 rows). When the
    output buffers are not given they are allocated zero-filled, so padding
    rows read back as zero. Returns (expand_x, expand_scales, expand_weights).
    """
    T = np.asarray(x_bytes).shape[0]
    xb = _byte_rows(x_bytes, T)
    row_bytes = xb.shape[1]
    dst = np.ascontiguousarray(dst_slot, dtype=np.int32)
    K = dst.shape[1]
    cap = int(capacity_rows)
    if expand_x is None:
        expand_x = np.zeros((cap, row_bytes), np.uint8)
    sb = 0
    xs = None
    if x_scales is not None:
        xs = _byte_rows(x_scales, T)
        sb = xs.shape[1]
        if expand_scales is None:
            expand_scales = np.zeros((cap, sb), np.uint8)
    w = None
    if topk_weights is not None:
        w = np.ascontiguousarray(topk_weights, dtype=np.float32)
        if expand_weights is None:
            expand_weights = np.zeros(cap, np.float32)
    ex = _byte_rows(expand_x, cap)
    es = None if expand_scales is None else _byte_rows(expand_scales, cap)
    rc = lib(_lib).oracle_dispatch(_ptr(xb, _u8p), row_bytes, _ptr(xs, _u8p), sb, _ptr(w, _f32p),
                               _ptr(dst, _i32p), T, K, cap, _ptr(ex, _u8p), _ptr(es, _u8p),
                               _ptr(expand_weights if w is not None else None, _f32p))
    if rc != 0:
        raise ValueError("oracle_dispatch rejected its arguments")
    return expand_x, expand_scales, expand_weights


def dispatch_compact(x_bytes: np.ndarray, topk_idx: np.ndarray, dst_slot: np.ndarray,
                     recv_src_metadata: np.ndarray, num_recv: int, x_scales: np.ndarray = None,
                     topk_weights: np.ndarray = None, _lib=None):
    """Non-expand dispatch: (recv_x bytes [num_recv, row_bytes], recv_scales bytes or None,
    recv_topk_idx int32 [num_recv, K], recv_topk_weights float32 or None)."""
    T = np.asarray(x_bytes).shape[0]
    xb = _byte_rows(x_bytes, T)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    dst = np.ascontiguousarray(dst_slot, dtype=np.int32)
    K = dst.shape[1]
    meta = np.ascontiguousarray(recv_src_metadata, dtype=np.int32).reshape(-1, K + 2)
    n = int(num_recv)
    rx = np.zeros((n, xb.shape[1]), np.uint8)
    xs = rs = None
    if x_scales is not None:
        xs = _byte_rows(x_scales, T)
        rs = np.zeros((n, xs.shape[1]), np.uint8)
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    ri = np.zeros((n, K), np.int32)
    rw = None if w is None else np.zeros((n, K), np.float32)
    rc = lib(_lib).oracle_dispatch_compact(_ptr(xb, _u8p), xb.shape[1], _ptr(xs, _u8p),
                                           0 if xs is None else xs.shape[1], _ptr(idx, _i32p),
                                           _ptr(w, _f32p), _ptr(dst, _i32p), _ptr(meta, _i32p), n, T, K,
                                           _ptr(rx, _u8p), _ptr(rs, _u8p), _ptr(ri, _i32p), _ptr(rw, _f32p))
    if rc != 0:
        raise ValueError("oracle_dispatch_compact rejected its arguments")
    return rx, rs, ri, rw


def combine_compact(y_bf16_bits: np.ndarray, dst_slot: np.ndarray, recv_src_metadata: np.ndarray,
                    num_recv: int, bias_bf16_bits: np.ndarray = None, _lib=None):
    """Non-expand combine: bf16 rows [>= num_recv, H] back to token order [T, H] (+ bias)."""
    y = np.ascontiguousarray(y_bf16_bits).view(np.uint16)
    H = y.shape[1]
    dst = np.ascontiguousarray(dst_slot, dtype=np.int32)
    T, K = dst.shape
    meta = np.ascontiguousarray(recv_src_metadata, dtype=np.int32).reshape(-1, K + 2)
    b = None if bias_bf16_bits is None else np.ascontiguousarray(bias_bf16_bits).view(np.uint16)
    out = np.empty((T, H), np.uint16)
    rc = lib(_lib).oracle_combine_compact(_ptr(y, _u16p), H, _ptr(b, _u16p), _ptr(dst, _i32p),
                                          _ptr(meta, _i32p), int(num_recv), T, K, _ptr(out, _u16p))
    if rc != 0:
        raise ValueError("oracle_combine_compact rejected its arguments")
    return out


def combine_compact_f32(y: np.ndarray, dst_slot: np.ndarray, recv_src_metadata: np.ndarray,
                        num_recv: int, bias: np.ndarray = None, _lib=None):
    """Non-expand combine of fp32 rows [>= num_recv, H] back to token order [T, H] (+ bias)."""
    yf = np.ascontiguousarray(y, dtype=np.float32)
    H = yf.shape[1]
    dst = np.ascontiguousarray(dst_slot, dtype=np.int32)
    T, K = dst.shape
    meta = np.ascontiguousarray(recv_src_metadata, dtype=np.int32).reshape(-1, K + 2)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, H), np.float32)
    rc = lib(_lib).oracle_combine_compact_f32(_ptr(yf, _f32p), H, _ptr(b, _f32p), _ptr(dst, _i32p),
                                              _ptr(meta, _i32p), int(num_recv), T, K,
                                              _ptr(out, _f32p))
    if rc != 0:
        raise ValueError("oracle_combine_compact_f32 rejected its arguments")
    return out


def zero_padding(expand_x: np.ndarray, counts: np.ndarray, offsets: np.ndarray,
                 expand_scales: np.ndarray = None, expand_weights: np.ndarray = None, _lib=None):
    """Zero the alignment padding rows of the expand buffers in place (and return them)."""
    cap = expand_x.shape[0]
    ex = _byte_rows(expand_x, cap)
    es = None if expand_scales is None else _byte_rows(expand_scales, cap)
    c = np.ascontiguousarray(counts, dtype=np.int32)
    o = np.ascontiguousarray(offsets, dtype=np.int32)
    rc = lib(_lib).oracle_zero_padding(_ptr(ex, _u8p), ex.shape[1], _ptr(es, _u8p),
                                       0 if es is None else es.shape[1], _ptr(expand_weights, _f32p),
                                       _ptr(c, _i32p), _ptr(o, _i32p), c.size, cap)
    if rc != 0:
        raise ValueError("oracle_zero_padding rejected its arguments")
    return expand_x, expand_scales, expand_weights


def combine(y_bf16_bits: np.ndarray, dst_slot: np.ndarray, topk_weights: np.ndarray = None,
            bias_bf16_bits: np.ndarray = None, _lib=None):
    """Weighted gather-reduce of bf16 expert outputs back to token order.

    ``y_bf16_bits`` is uint16 [capacity, H] holding bf16 bit patterns, the
    optional bias uint16 [T, H]; returns uint16 [T, H] bf16 bit patterns.
    """
    y = np.ascontiguousarray(y_bf16_bits).view(np.uint16)
    cap, H = y.shape
    dst = np.ascontiguousarray(dst_slot, dtype=np.int32)
    T, K = dst.shape
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    b = None if bias_bf16_bits is None else np.ascontiguousarray(bias_bf16_bits).view(np.uint16)
    out = np.empty((T, H), np.uint16)
    rc = lib(_lib).oracle_combine(_ptr(y, _u16p), H, _ptr(w, _f32p), _ptr(b, _u16p),
                                  _ptr(dst, _i32p), T, K, cap, _ptr(out, _u16p))
    if rc != 0:
        raise ValueError("oracle_combine rejected its arguments")
    return out


def combine_f32(y: np.ndarray, dst_slot: np.ndarray, topk_weights: np.ndarray = None,
                bias: np.ndarray = None, _lib=None):
    """Weighted gather-reduce of fp32 expert outputs [capacity, H] into fp32 [T, H]."""
    yf = np.ascontiguousarray(y, dtype=np.float32)
    cap, H = yf.shape
    dst = np.ascontiguousarray(dst_slot, dtype=np.int32)
    T, K = dst.shape
    w = None if topk_weights is None else np.ascontiguousarray(topk_weights, dtype=np.float32)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty((T, H), np.float32)
    rc = lib(_lib).oracle_combine_f32(_ptr(yf, _f32p), H, _ptr(w, _f32p), _ptr(b, _f32p),
                                      _ptr(dst, _i32p), T, K, cap, _ptr(out, _f32p))
    if rc != 0:
        raise ValueError("oracle_combine_f32 rejected its arguments")
    return out


def f32_to_bf16(f: float, _lib=None) -> int:
    """The oracle's binary32 -> bf16 rounding (round to nearest even)."""
    return int(lib(_lib).oracle_f32_to_bf16(float(f)))


def bf16_to_f32(b: int, _lib=None) -> float:
    return float(lib(_lib).oracle_bf16_to_f32(int(b)))
