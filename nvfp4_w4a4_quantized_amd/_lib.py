"""ctypes binding of libnvfp4moe.so (the C ABI in include/nvfp4moe.h).

Argument marshalling only: every step of the path runs in the library's gfx950
kernels.  torch supplies device memory and the current HIP stream.  Loading
fails loudly when the library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4moe.so")
# the same library built with NVFP4_DEBUG_CHECKS (device-side precondition
# checks reported in the workspace's precondition word)
DEBUG_LIB_PATH = os.path.join(_HERE, "libnvfp4moe_debug.so")

_vp = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32


class NvFp4Error(RuntimeError):
    pass


class Weights(C.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp), ("gscale", _vp), ("layout", C.c_int32)]


class Intermediates(C.Structure):
    _fields_ = [(n, _vp) for n in (
        "expert_offsets", "dst_row", "row_src", "row_prob", "a1_codes", "a1_scales", "a1_gscale",
        "fc1_out", "d", "amax_d", "a2_codes", "a2_scales", "a2_gscale", "y_rows", "y_rows_f32")]


class SinglePassIntermediates(C.Structure):
    _fields_ = [(n, _vp) for n in (
        "expert_offsets", "dst_row", "row_src", "row_prob", "a1_codes", "a1_scales", "a1_gscale",
        "fc1_out", "p", "a2_codes", "a2_scales", "gs_tiles", "y_rows", "y_rows_f32")]


class BackwardIntermediates(C.Structure):
    _fields_ = [(n, _vp) for n in ("dd", "dc", "dp_rows", "dx_rows", "dx_rows_f32")]


_lib = None
_debug_lib = None


def lib():
    """The release library (loaded once)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib():
    """The NVFP4_DEBUG_CHECKS build of the same interface (loaded once)."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def _load(path):
    if not os.path.exists(path):
        raise NvFp4Error(f"{path} is missing: build it with `python -m "
                         "nvfp4_w4a4_quantized_amd.build` (there is no fallback path)")
    L = C.CDLL(path)
    L.nvfp4_debug_checks.restype = C.c_int
    L.nvfp4_debug_checks.argtypes = []
    L.nvfp4_status_string.restype = C.c_char_p
    L.nvfp4_status_string.argtypes = [C.c_int]
    L.nvfp4_quantize.restype = C.c_int
    L.nvfp4_quantize.argtypes = [_vp, _i64, _i64, _i64, C.c_int, _vp, _i32, _vp, C.c_int, _vp, _vp,
                                 _vp, _vp]
    L.moe_rows_capacity.restype = _i64
    L.moe_rows_capacity.argtypes = [_i64, _i32, _i32, _i32]
    L.moe_permute_workspace_size.restype = C.c_size_t
    L.moe_permute_workspace_size.argtypes = [_i64, _i32, _i32]
    L.moe_permute.restype = C.c_int
    L.moe_permute.argtypes = [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                              _vp, _vp, _vp, _vp, _vp, C.c_size_t, _vp]
    L.moe_permute_noalloc.restype = C.c_int
    L.moe_permute_noalloc.argtypes = [_vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp]
    L.w4a4_grouped_gemm.restype = C.c_int
    L.w4a4_grouped_gemm.argtypes = [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i64, _i64,
                                    C.c_int, C.c_int, _vp, _vp]
    L.w4a4_grouped_gemm_swiglu.restype = C.c_int
    L.w4a4_grouped_gemm_swiglu.argtypes = [_vp, _vp, _vp, _i64, _vp, _vp, _vp, _vp, _i32, _i64,
                                           _i64, C.c_int, _vp, _vp, _vp, _vp, _vp]
    L.nvfp4_pack_weights.restype = C.c_int
    L.nvfp4_pack_weights.argtypes = [_vp, _vp, _i32, _i64, _i64, _vp, _vp, _vp]
    L.moe_combine.restype = C.c_int
    L.moe_combine.argtypes = [_vp, C.c_int, _vp, _i64, _i32, _i64, _vp, _vp]
    L.moe_expert_forward_workspace_size.restype = C.c_size_t
    L.moe_expert_forward_workspace_size.argtypes = [_i64, _i64, _i64, _i32, _i32, _i32]
    L.moe_expert_forward.restype = C.c_int
    L.moe_expert_forward.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i32, _i32, _i32, _i32,
                                     _i32, C.POINTER(Weights), C.POINTER(Weights), _vp, _vp,
                                     C.c_size_t,
                                     C.POINTER(Intermediates), _vp, _vp]
    L.moe_expert_forward_single_pass_workspace_size.restype = C.c_size_t
    L.moe_expert_forward_single_pass_workspace_size.argtypes = [_i64, _i64, _i64, _i32, _i32, _i32]
    L.moe_expert_forward_single_pass.restype = C.c_int
    L.moe_expert_forward_single_pass.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i32, _i32,
                                                 _i32, C.POINTER(Weights), C.POINTER(Weights),
                                                 _vp, _vp, C.c_size_t,
                                                 C.POINTER(SinglePassIntermediates), _vp, _vp]
    L.moe_expert_backward_workspace_size.restype = C.c_size_t
    L.moe_expert_backward_workspace_size.argtypes = [_i64, _i64, _i64, _i32]
    L.moe_expert_backward.restype = C.c_int
    L.moe_expert_backward.argtypes = [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _i64, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      C.c_size_t, C.POINTER(BackwardIntermediates), _vp, _vp]
    L.nvfp4_event_create.restype = C.c_int
    L.nvfp4_event_create.argtypes = [C.POINTER(_vp)]
    L.nvfp4_event_record.restype = C.c_int
    L.nvfp4_event_record.argtypes = [_vp, _vp]
    L.nvfp4_event_elapsed_ms.restype = C.c_int
    L.nvfp4_event_elapsed_ms.argtypes = [_vp, _vp, C.POINTER(C.c_float)]
    L.nvfp4_event_destroy.restype = C.c_int
    L.nvfp4_event_destroy.argtypes = [_vp]
    return L


def check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().nvfp4_status_string(status).decode()
        raise NvFp4Error(f"{what}: {msg} (status {status})")


def ptr(t):
    """Device address of a tensor (None -> NULL)."""
    if t is None:
        return None
    return _vp(t.data_ptr())


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return _vp(s.cuda_stream)
