"""Thin ctypes binding of libep_mi355x.so (argument marshalling only).

The functions carry the C ABI's names and arguments (see
include/ep_mi355x.h). Array arguments may be anything with ``data_ptr()``
(a torch tensor on the GPU), a raw device address (int) or None; ``stream``
may be a torch stream (``.cuda_stream``), a raw hipStream_t (int) or None
for the default stream. Every step of the path runs in the library's HIP
kernels; this module never computes anything and never falls back to
another implementation: if the library is missing it raises. The
environment variable EP_MI355X_LIB names another build of the same library
to load instead (for example the host-sanitized libep_mi355x_asan.so).
"""
import ctypes
import os

LIB_PATH = (os.environ.get("EP_MI355X_LIB")
            or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libep_mi355x.so"))

EP_OK = 0
EP_EINVAL = -1
EP_EUNSUPPORTED = -2
EP_ECAPACITY = -3
EP_EHIP = -4

EP_BF16 = 0
EP_FP32 = 1
EP_FP8_E4M3 = 2
EP_FP4X2 = 3

EP_MAX_EXPERTS = 1024
EP_MAX_TOPK = 64
EP_LAYOUT_SCRATCH_BYTES = 8 << 20

SYMBOLS = ("ep_layout_workspace_bytes", "ep_layout", "ep_dispatch", "ep_layout_dispatch",
           "ep_combine",
           "ep_dispatch_compact", "ep_layout_dispatch_compact", "ep_combine_compact",
           "ep_zero_padding", "ep_set_workgroup_limit",
           "ep_get_workgroup_limit", "ep_last_error", "ep_supported", "ep_layout_noalloc",
           "ep_layout_dispatch_workspace_bytes")


class EpError(RuntimeError):
    """A negative return code from the C ABI, with ep_last_error()'s message."""

    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


_LIB = None

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


def lib(path: str = None) -> ctypes.CDLL:
    """Load the C-ABI library; raise if it has not been built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build the HIP library first "
                          "(python -m combine_ep_layout_amd.build, or __graft_entry__.build())")
    L = ctypes.CDLL(p)
    L.ep_layout_workspace_bytes.argtypes = [_i32, _i32, _i32]
    L.ep_layout_workspace_bytes.restype = _sz
    L.ep_layout_dispatch_workspace_bytes.argtypes = [_i32, _i32, _i32]
    L.ep_layout_dispatch_workspace_bytes.restype = _sz
    L.ep_layout.argtypes = [_vp, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
                            _vp, _sz, _vp]
    L.ep_layout.restype = ctypes.c_int
    L.ep_layout_noalloc.argtypes = [_vp, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _sz, _vp]
    L.ep_layout_noalloc.restype = ctypes.c_int
    L.ep_dispatch.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp,
                              _vp]
    L.ep_dispatch.restype = ctypes.c_int
    L.ep_layout_dispatch.argtypes = [_vp, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _sz, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]
    L.ep_layout_dispatch.restype = ctypes.c_int
    L.ep_combine.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i64, _vp, _vp]
    L.ep_combine.restype = ctypes.c_int
    L.ep_dispatch_compact.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                      _vp, _vp, _vp, _vp, _vp]
    L.ep_dispatch_compact.restype = ctypes.c_int
    L.ep_layout_dispatch_compact.argtypes = [_vp, _i32, _i32, _i32, _i32, _i64, _vp, _vp, _vp, _vp,
                                             _vp, _vp, _sz, _vp, _vp, _vp, _i32, _i32, _vp, _vp,
                                             _vp, _vp, _vp]
    L.ep_layout_dispatch_compact.restype = ctypes.c_int
    L.ep_combine_compact.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp]
    L.ep_combine_compact.restype = ctypes.c_int
    L.ep_set_workgroup_limit.argtypes = [_vp, _i32]
    L.ep_set_workgroup_limit.restype = ctypes.c_int
    L.ep_get_workgroup_limit.argtypes = [_vp]
    L.ep_get_workgroup_limit.restype = ctypes.c_int
    L.ep_zero_padding.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _i32, _i64, _vp]
    L.ep_zero_padding.restype = ctypes.c_int
    L.ep_last_error.argtypes = []
    L.ep_last_error.restype = ctypes.c_char_p
    L.ep_supported.argtypes = [_i32, _i32, _i32, _i32]
    L.ep_supported.restype = ctypes.c_int
    if path is None:
        _LIB = L
    return L


def use_library(path: str = None) -> ctypes.CDLL:
    """Make the module's functions call the library at `path` (another build of the same
    library, as EP_MI355X_LIB does at import), or the default one for None; returns it."""
    global _LIB
    _LIB = None
    L = lib(path or LIB_PATH)
    _LIB = L
    return L


def _p(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if hasattr(a, "is_contiguous") and not a.is_contiguous():
        raise ValueError("arrays passed to the C ABI must be contiguous")
    return a.data_ptr()


def _s(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int):
    if rc != EP_OK:
        raise EpError(rc, lib().ep_last_error().decode(errors="replace"))


def ep_last_error() -> str:
    return lib().ep_last_error().decode(errors="replace")


def ep_supported(pass_: int, hidden: int, topk: int, dtype: int) -> bool:
    return bool(lib().ep_supported(pass_, hidden, topk, dtype))


def ep_layout_workspace_bytes(num_tokens: int, topk: int, num_experts: int) -> int:
    return int(lib().ep_layout_workspace_bytes(num_tokens, topk, num_experts))


def _nbytes(a, nbytes):
    """Byte count of an optional read-ahead region: given, else the tensor's own size."""
    if a is None:
        return 0
    return int(a.nbytes) if nbytes is None else int(nbytes)


def ep_layout_dispatch_workspace_bytes(num_tokens: int, topk: int, num_experts: int) -> int:
    return int(lib().ep_layout_dispatch_workspace_bytes(num_tokens, topk, num_experts))


def ep_layout(topk_idx, num_tokens, topk, num_experts, expert_alignment, capacity_rows,
              counts, offsets, dst_slot, recv_src_metadata, num_recv, workspace,
              workspace_bytes, stream=None, dispatch_plan=None, prefetch=None,
              prefetch_bytes=None):
    _check(lib().ep_layout(_p(topk_idx), num_tokens, topk, num_experts, expert_alignment,
                           capacity_rows, _p(counts), _p(offsets), _p(dst_slot),
                           _p(recv_src_metadata), _p(num_recv), _p(workspace),
                           workspace_bytes, _p(dispatch_plan), _p(prefetch),
                           _nbytes(prefetch, prefetch_bytes), _s(stream)))


def ep_layout_noalloc(topk_idx, num_tokens, topk, num_experts, expert_alignment, capacity_rows,
                      counts, offsets, dst_slot, recv_src_metadata, num_recv, stream=None,
                      dispatch_plan=None, prefetch=None, prefetch_bytes=None):
    _check(lib().ep_layout_noalloc(_p(topk_idx), num_tokens, topk, num_experts, expert_alignment,
                                   capacity_rows, _p(counts), _p(offsets), _p(dst_slot),
                                   _p(recv_src_metadata), _p(num_recv), _p(dispatch_plan),
                                   _p(prefetch), _nbytes(prefetch, prefetch_bytes), _s(stream)))


def ep_dispatch(x, x_scales, topk_weights, dst_slot, num_tokens, hidden, topk, dtype,
                capacity_rows, expand_x, expand_scales, expand_weights, stream=None,
                dispatch_plan=None):
    _check(lib().ep_dispatch(_p(x), _p(x_scales), _p(topk_weights), _p(dst_slot), num_tokens,
                             hidden, topk, dtype, capacity_rows, _p(expand_x), _p(expand_scales),
                             _p(expand_weights), _p(dispatch_plan), _s(stream)))


def ep_layout_dispatch(topk_idx, num_tokens, topk, num_experts, expert_alignment, capacity_rows,
                       counts, offsets, dst_slot, recv_src_metadata, num_recv, workspace,
                       workspace_bytes, x, x_scales, topk_weights, hidden, dtype, expand_x,
                       expand_scales, expand_weights, stream=None):
    _check(lib().ep_layout_dispatch(_p(topk_idx), num_tokens, topk, num_experts, expert_alignment,
                                    capacity_rows, _p(counts), _p(offsets), _p(dst_slot),
                                    _p(recv_src_metadata), _p(num_recv), _p(workspace),
                                    workspace_bytes, _p(x), _p(x_scales), _p(topk_weights), hidden,
                                    dtype, _p(expand_x), _p(expand_scales), _p(expand_weights),
                                    _s(stream)))


def ep_combine(expert_out, topk_weights, bias, dst_slot, num_tokens, hidden, topk, dtype,
               capacity_rows, out, stream=None):
    _check(lib().ep_combine(_p(expert_out), _p(topk_weights), _p(bias), _p(dst_slot), num_tokens,
                            hidden, topk, dtype, capacity_rows, _p(out), _s(stream)))


def ep_zero_padding(expand_x, row_bytes, expand_scales, scale_cols, expand_weights, counts, offsets,
                    num_experts, expert_alignment, capacity_rows, stream=None):
    _check(lib().ep_zero_padding(_p(expand_x), row_bytes, _p(expand_scales), scale_cols,
                                 _p(expand_weights), _p(counts), _p(offsets), num_experts,
                                 expert_alignment, capacity_rows, _s(stream)))


def ep_dispatch_compact(x, x_scales, topk_idx, topk_weights, dst_slot, recv_src_metadata, num_recv,
                        num_tokens, hidden, topk, dtype, recv_x, recv_scales, recv_topk_idx,
                        recv_topk_weights, stream=None):
    _check(lib().ep_dispatch_compact(_p(x), _p(x_scales), _p(topk_idx), _p(topk_weights),
                                     _p(dst_slot), _p(recv_src_metadata), _p(num_recv), num_tokens,
                                     hidden, topk, dtype, _p(recv_x), _p(recv_scales),
                                     _p(recv_topk_idx), _p(recv_topk_weights), _s(stream)))


def ep_layout_dispatch_compact(topk_idx, num_tokens, topk, num_experts, expert_alignment,
                               capacity_rows, counts, offsets, dst_slot, recv_src_metadata,
                               num_recv, workspace, workspace_bytes, x, x_scales, topk_weights,
                               hidden, dtype, recv_x, recv_scales, recv_topk_idx,
                               recv_topk_weights, stream=None):
    _check(lib().ep_layout_dispatch_compact(
        _p(topk_idx), num_tokens, topk, num_experts, expert_alignment, capacity_rows, _p(counts),
        _p(offsets), _p(dst_slot), _p(recv_src_metadata), _p(num_recv), _p(workspace),
        workspace_bytes, _p(x), _p(x_scales), _p(topk_weights), hidden, dtype, _p(recv_x),
        _p(recv_scales), _p(recv_topk_idx), _p(recv_topk_weights), _s(stream)))


def ep_combine_compact(expert_out, bias, dst_slot, recv_src_metadata, num_recv, num_tokens, hidden,
                       topk, dtype, out, stream=None):
    _check(lib().ep_combine_compact(_p(expert_out), _p(bias), _p(dst_slot), _p(recv_src_metadata),
                                    _p(num_recv), num_tokens, hidden, topk, dtype, _p(out),
                                    _s(stream)))


def ep_set_workgroup_limit(stream, max_workgroups):
    _check(lib().ep_set_workgroup_limit(_s(stream), max_workgroups))


def ep_get_workgroup_limit(stream) -> int:
    return lib().ep_get_workgroup_limit(_s(stream))
