"""ctypes binding of the CPU oracle (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this module.  It takes and returns numpy arrays
(bf16 travels as ``uint16`` bit patterns) and shares nothing with the HIP
library.  The definitions it computes are documented in ``nvfp4_oracle.h``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_libs = {}

_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


class _MoeBuffers(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "a1_codes", "a1_scales", "a1_gscale", "c_fc1", "d", "amax_d",
        "a2_codes", "a2_scales", "a2_gscale", "y_rows",
        "offsets", "dst_row", "row_src", "row_prob")]


_override = None


def use_library(path):
    """Routes every function of this module to the oracle library at `path`
    (None restores the default).  Used by the planted-mistake tests."""
    global _override
    _override = path


def lib():
    """Loads liboracle.so (or the library chosen by use_library)."""
    path = _override or _LIB_PATH
    if path in _libs:
        return _libs[path]
    if path == _LIB_PATH and not os.path.exists(_LIB_PATH):
        from . import build as _build  # build on demand
        _build.build()
    L = C.CDLL(path)
    L.orc_e2m1_value.restype = C.c_double
    L.orc_e2m1_value.argtypes = [C.c_uint]
    L.orc_e2m1_encode.restype = C.c_uint
    L.orc_e2m1_encode.argtypes = [C.c_float]
    L.orc_e4m3_value.restype = C.c_double
    L.orc_e4m3_value.argtypes = [C.c_uint]
    L.orc_e4m3_encode.restype = C.c_uint
    L.orc_e4m3_encode.argtypes = [C.c_float]
    L.orc_f64_to_bf16.restype = C.c_uint16
    L.orc_f64_to_bf16.argtypes = [C.c_double]
    L.orc_row_amax.restype = C.c_float
    L.orc_row_amax.argtypes = [_u16p, C.c_int64]
    L.orc_quantize.restype = C.c_int
    L.orc_quantize.argtypes = [_u16p, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_void_p,
                               C.c_int32, C.c_void_p, _u8p, _u8p, _f32p]
    L.orc_quantize_rule.restype = C.c_int
    L.orc_quantize_rule.argtypes = [_u16p, C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_void_p,
                                    C.c_int32, C.c_void_p, C.c_int, _u8p, _u8p, _f32p]
    L.orc_outer_scale.restype = C.c_float
    L.orc_outer_scale.argtypes = [C.c_float, C.c_int]
    L.orc_dequantize_row.restype = None
    L.orc_dequantize_row.argtypes = [_u8p, _u8p, C.c_float, C.c_int64, _f64p]
    L.orc_rows_capacity.restype = C.c_int64
    L.orc_rows_capacity.argtypes = [C.c_int64, C.c_int32, C.c_int32, C.c_int32]
    L.orc_route.restype = C.c_int
    L.orc_route.argtypes = [_i32p, _f32p, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                            _i32p, _i32p, _i32p, _f32p]
    L.orc_moe_permute.restype = C.c_int
    L.orc_moe_permute.argtypes = [C.c_void_p, C.c_int64, C.c_int64, _i32p, _f32p, C.c_int32,
                                  C.c_int32, C.c_int32, _i32p, _i32p, _i32p, _f32p,
                                  C.c_void_p, C.c_void_p, C.c_void_p]
    L.orc_moe_permute_rule.restype = C.c_int
    L.orc_moe_permute_rule.argtypes = [C.c_void_p, C.c_int64, C.c_int64, _i32p, _f32p, C.c_int32,
                                       C.c_int32, C.c_int32, C.c_int, _i32p, _i32p, _i32p, _f32p,
                                       C.c_void_p, C.c_void_p, C.c_void_p]
    L.orc_grouped_gemm.restype = C.c_int
    L.orc_grouped_gemm.argtypes = [_u8p, _u8p, _f32p, _u8p, _u8p, _f32p, _i32p, C.c_int32,
                                   C.c_int64, C.c_int64, _f32p, C.c_void_p]
    L.orc_grouped_gemm_at.restype = C.c_int
    L.orc_grouped_gemm_at.argtypes = [_u8p, _u8p, _f32p, _u8p, _u8p, _f32p, _i32p, C.c_int32,
                                      C.c_int64, C.c_int64, _i64p, _i64p, C.c_int64, _f32p,
                                      C.c_void_p]
    L.orc_swiglu.restype = None
    L.orc_swiglu.argtypes = [_f32p, _f32p, C.c_int64, C.c_int64, _u16p, _f32p]
    L.orc_combine.restype = None
    L.orc_combine.argtypes = [_f32p, _i32p, C.c_int64, C.c_int32, C.c_int64, _u16p]
    L.orc_moe_forward.restype = C.c_int
    L.orc_moe_forward.argtypes = [_u16p, C.c_int64, C.c_int64, C.c_int64, _i32p, _f32p,
                                  C.c_int32, C.c_int32, C.c_int32,
                                  _u8p, _u8p, _f32p, _u8p, _u8p, _f32p,
                                  C.POINTER(_MoeBuffers), _u16p, C.c_void_p]
    L.orc_moe_forward_rule.restype = C.c_int
    L.orc_moe_forward_rule.argtypes = [_u16p, C.c_int64, C.c_int64, C.c_int64, _i32p, _f32p,
                                       C.c_int32, C.c_int32, C.c_int32, C.c_int,
                                       _u8p, _u8p, _f32p, _u8p, _u8p, _f32p,
                                       C.POINTER(_MoeBuffers), _u16p, C.c_void_p]
    L.orc_online_quantize.restype = C.c_int
    L.orc_online_quantize.argtypes = [_u16p, C.c_int64, C.c_int64, C.c_int64, _u8p, _u8p, _f32p]
    L.orc_single_pass_gemm.restype = C.c_int
    L.orc_single_pass_gemm.argtypes = [_u8p, _u8p, _f32p, C.c_int64, _u8p, _u8p, _f32p, _i32p,
                                       C.c_int32, C.c_int64, C.c_int64, _f32p, C.c_void_p]
    L.orc_moe_forward_single_pass.restype = C.c_int
    L.orc_moe_forward_single_pass.argtypes = [_u16p, C.c_int64, C.c_int64, C.c_int64, _i32p,
                                              _f32p, C.c_int32, C.c_int32, C.c_int32, C.c_int64,
                                              _u8p, _u8p, _f32p, _u8p, _u8p, _f32p,
                                              C.POINTER(_MoeBuffers), _f32p, _u16p, C.c_void_p]
    L.orc_num_threads.restype = C.c_int
    L.orc_num_threads.argtypes = []
    L.orc_set_num_threads.restype = None
    L.orc_set_num_threads.argtypes = [C.c_int]
    _libs[path] = L
    return L


def _check(status: int, what: str) -> None:
    if status != 0:
        raise ValueError(f"oracle {what}: invalid argument (status {status})")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


# ---- scalar codecs --------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(code)


def e2m1_encode(r: float) -> int:
    return lib().orc_e2m1_encode(r)


def e4m3_value(byte: int) -> float:
    return lib().orc_e4m3_value(byte)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def f64_to_bf16(v: float) -> int:
    return lib().orc_f64_to_bf16(v)


def set_num_threads(n: int) -> None:
    """Threads of the following oracle calls (the results do not depend on it)."""
    lib().orc_set_num_threads(int(n))


def num_threads() -> int:
    return lib().orc_num_threads()


# ---- quantization ---------------------------------------------------------

def outer_scale(amax: float, rule: int = 0) -> float:
    return lib().orc_outer_scale(amax, rule)


def quantize(x_bf16: np.ndarray, domain: int = 0, group_offsets=None, amax_in=None, rule: int = 0):
    """NVFP4 quantization of a bf16 [rows, k] matrix (uint16 bit patterns).

    Returns (codes u8 [rows, k/2], scales u8 [rows, k/16], gscale f32 [rows] or
    [groups]).
    """
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, k = x.shape
    codes = np.zeros((rows, k // 2), np.uint8)
    scales = np.zeros((rows, k // 16), np.uint8)
    if domain == 0:
        ng, offs = 0, None
        gscale = np.zeros(rows, np.float32)
    else:
        offs = np.ascontiguousarray(group_offsets, dtype=np.int32)
        ng = offs.size - 1
        gscale = np.zeros(ng, np.float32)
    am = None if amax_in is None else np.ascontiguousarray(amax_in, dtype=np.float32)
    if rule == 0:
        _check(lib().orc_quantize(x, rows, k, k, domain, _ptr(offs), ng, _ptr(am),
                                  codes, scales, gscale), "quantize")
    else:
        _check(lib().orc_quantize_rule(x, rows, k, k, domain, _ptr(offs), ng, _ptr(am), rule,
                                       codes, scales, gscale), "quantize")
    return codes, scales, gscale


def dequantize(codes: np.ndarray, scales: np.ndarray, gscale_rows: np.ndarray) -> np.ndarray:
    """x^ = q * s_b * s_g (fp64) for every row; gscale_rows holds one s_g per row."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    rows = codes.shape[0]
    k = codes.shape[1] * 2
    out = np.zeros((rows, k), np.float64)
    g = np.ascontiguousarray(gscale_rows, np.float32)
    L = lib()
    for r in range(rows):
        row = np.zeros(k, np.float64)
        L.orc_dequantize_row(np.ascontiguousarray(codes[r]), np.ascontiguousarray(scales[r]),
                             float(g[r]), k, row)
        out[r] = row
    return out


# ---- routing --------------------------------------------------------------

def rows_capacity(tokens: int, topk: int, num_experts: int, align: int = 1) -> int:
    return int(lib().orc_rows_capacity(tokens, topk, num_experts, align))


def route(topk_idx: np.ndarray, topk_prob: np.ndarray, num_experts: int, align: int = 1):
    idx = np.ascontiguousarray(topk_idx, np.int32)
    prob = np.ascontiguousarray(topk_prob, np.float32)
    T, k = idx.shape
    cap = rows_capacity(T, k, num_experts, align)
    offsets = np.zeros(num_experts + 1, np.int32)
    dst = np.zeros((T, k), np.int32)
    src = np.full(cap, -2, np.int32)
    rp = np.full(cap, np.nan, np.float32)
    _check(lib().orc_route(idx, prob, T, k, num_experts, align, offsets, dst, src, rp), "route")
    return offsets, dst, src, rp


def moe_permute(x_bf16, topk_idx, topk_prob, num_experts: int, align: int = 1, rule: int = 0):
    """Route + per-token quantize-scatter.  Returns a dict of numpy arrays."""
    idx = np.ascontiguousarray(topk_idx, np.int32)
    prob = np.ascontiguousarray(topk_prob, np.float32)
    T, k = idx.shape
    cap = rows_capacity(T, k, num_experts, align)
    offsets = np.zeros(num_experts + 1, np.int32)
    dst = np.zeros((T, k), np.int32)
    src = np.full(cap, -2, np.int32)
    rp = np.full(cap, np.nan, np.float32)
    if x_bf16 is None:
        _check(lib().orc_moe_permute(None, T, 0, idx, prob, k, num_experts, align,
                                     offsets, dst, src, rp, None, None, None), "moe_permute")
        return dict(offsets=offsets, dst_row=dst, row_src=src, row_prob=rp)
    x = np.ascontiguousarray(x_bf16, np.uint16)
    H = x.shape[1]
    codes = np.zeros((cap, H // 2), np.uint8)
    scales = np.zeros((cap, H // 16), np.uint8)
    gs = np.zeros(cap, np.float32)
    _check(lib().orc_moe_permute_rule(_ptr(x), T, H, idx, prob, k, num_experts, align, rule,
                                      offsets, dst, src, rp, _ptr(codes), _ptr(scales), _ptr(gs)),
           "moe_permute")
    return dict(offsets=offsets, dst_row=dst, row_src=src, row_prob=rp,
                codes=codes, scales=scales, gscale=gs)


# ---- GEMM -----------------------------------------------------------------

def grouped_gemm(a_codes, a_scales, a_gscale, b_codes, b_scales, b_gscale, offsets,
                 with_bound: bool = False):
    """Full grouped GEMM (fp32 result, fp64 bound).  B is [G, N, K/2]."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    rows, kh = a_codes.shape
    G, n, _ = b_codes.shape
    out = np.zeros((rows, n), np.float32)
    bound = np.zeros((rows, n), np.float64) if with_bound else None
    _check(lib().orc_grouped_gemm(a_codes, np.ascontiguousarray(a_scales, np.uint8),
                                  np.ascontiguousarray(a_gscale, np.float32),
                                  np.ascontiguousarray(b_codes, np.uint8),
                                  np.ascontiguousarray(b_scales, np.uint8),
                                  np.ascontiguousarray(b_gscale, np.float32),
                                  np.ascontiguousarray(offsets, np.int32), G, n, kh * 2, out,
                                  _ptr(bound)), "grouped_gemm")
    return (out, bound) if with_bound else out


def grouped_gemm_at(a_codes, a_scales, a_gscale, b_codes, b_scales, b_gscale, offsets,
                    rows, cols):
    """The grouped GEMM definition evaluated at (rows[i], cols[i]) only.

    Returns (values f32, bound f64)."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    kh = a_codes.shape[1]
    G, n, _ = b_codes.shape
    rows = np.ascontiguousarray(rows, np.int64)
    cols = np.ascontiguousarray(cols, np.int64)
    out = np.zeros(rows.size, np.float32)
    bound = np.zeros(rows.size, np.float64)
    _check(lib().orc_grouped_gemm_at(a_codes, np.ascontiguousarray(a_scales, np.uint8),
                                     np.ascontiguousarray(a_gscale, np.float32),
                                     np.ascontiguousarray(b_codes, np.uint8),
                                     np.ascontiguousarray(b_scales, np.uint8),
                                     np.ascontiguousarray(b_gscale, np.float32),
                                     np.ascontiguousarray(offsets, np.int32), G, n, kh * 2,
                                     rows, cols, rows.size, out, _ptr(bound)),
           "grouped_gemm_at")
    return out, bound


# ---- SwiGLU / combine ---------------------------------------------------

def swiglu(c_fc1: np.ndarray, prob: np.ndarray):
    c = np.ascontiguousarray(c_fc1, np.float32)
    rows, n2 = c.shape
    inter = n2 // 2
    d = np.zeros((rows, inter), np.uint16)
    amax = np.zeros(rows, np.float32)
    lib().orc_swiglu(c, np.ascontiguousarray(prob, np.float32), rows, inter, d, amax)
    return d, amax


def combine(y_rows: np.ndarray, dst_row: np.ndarray):
    yr = np.ascontiguousarray(y_rows, np.float32)
    dst = np.ascontiguousarray(dst_row, np.int32)
    T, k = dst.shape
    H = yr.shape[1]
    y = np.zeros((T, H), np.uint16)
    lib().orc_combine(yr, dst, T, k, H, y)
    return y


# ---- whole layer ----------------------------------------------------------

def moe_forward(x_bf16, topk_idx, topk_prob, num_experts, inter, w1, w2, align: int = 1,
                stage_times: bool = False, act_rule: int = 0):
    """Whole expert layer.  w1 / w2 are (codes, scales, gscale) NVFP4 triples with
    shapes [E, 2I, H/2] ... and [E, H, I/2] ....  Returns (y bf16 [T, H], dict of
    intermediates[, stage seconds])."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    idx = np.ascontiguousarray(topk_idx, np.int32)
    prob = np.ascontiguousarray(topk_prob, np.float32)
    T, H = x.shape
    k = idx.shape[1]
    I = inter
    cap = rows_capacity(T, k, num_experts, align)
    b = dict(
        a1_codes=np.zeros((cap, H // 2), np.uint8), a1_scales=np.zeros((cap, H // 16), np.uint8),
        a1_gscale=np.zeros(cap, np.float32), c_fc1=np.zeros((cap, 2 * I), np.float32),
        d=np.zeros((cap, I), np.uint16), amax_d=np.zeros(cap, np.float32),
        a2_codes=np.zeros((cap, I // 2), np.uint8), a2_scales=np.zeros((cap, I // 16), np.uint8),
        a2_gscale=np.zeros(cap, np.float32), y_rows=np.zeros((cap, H), np.float32),
        offsets=np.zeros(num_experts + 1, np.int32), dst_row=np.zeros((T, k), np.int32),
        row_src=np.zeros(cap, np.int32), row_prob=np.zeros(cap, np.float32))
    st = _MoeBuffers(**{n: b[n].ctypes.data for n in b})
    y = np.zeros((T, H), np.uint16)
    secs = np.zeros(6, np.float64)
    w1c, w1s, w1g = (np.ascontiguousarray(a) for a in w1)
    w2c, w2s, w2g = (np.ascontiguousarray(a) for a in w2)
    _check(lib().orc_moe_forward_rule(x, T, H, I, idx, prob, k, num_experts, align, act_rule,
                                 w1c.astype(np.uint8, copy=False), w1s.astype(np.uint8, copy=False),
                                 w1g.astype(np.float32, copy=False),
                                 w2c.astype(np.uint8, copy=False), w2s.astype(np.uint8, copy=False),
                                 w2g.astype(np.float32, copy=False),
                                 C.byref(st), y, secs.ctypes.data_as(C.c_void_p)), "moe_forward")
    if stage_times:
        return y, b, secs
    return y, b


# ---- O12: single-pass FC1 -> SwiGLU -> quantize -> FC2 ------------------

def num_tiles(inter: int, tile: int) -> int:
    return (inter + tile - 1) // tile


def online_quantize(p_bf16, tile: int):
    """O12a: tile-by-tile quantization of bf16 rows [rows, inter] with a
    running row amax.  Returns (codes, scales, gs [rows, ntiles])."""
    p = np.ascontiguousarray(p_bf16, np.uint16)
    rows, inter = p.shape
    codes = np.zeros((rows, inter // 2), np.uint8)
    scales = np.zeros((rows, inter // 16), np.uint8)
    gs = np.zeros((rows, num_tiles(inter, tile)), np.float32)
    _check(lib().orc_online_quantize(p, rows, inter, tile, codes, scales, gs), "online_quantize")
    return codes, scales, gs


def single_pass_gemm(a_codes, a_scales, gs, tile: int, b_codes, b_scales, b_gscale, offsets,
                     with_bound: bool = False):
    """O12b: the FC2 of online-quantized rows with the rescale of the
    partial sums at every tile (fp32 result, fp64 bound)."""
    a_codes = np.ascontiguousarray(a_codes, np.uint8)
    rows, kh = a_codes.shape
    G, n, _ = b_codes.shape
    out = np.zeros((rows, n), np.float32)
    bound = np.zeros((rows, n), np.float64) if with_bound else None
    _check(lib().orc_single_pass_gemm(a_codes, np.ascontiguousarray(a_scales, np.uint8),
                                      np.ascontiguousarray(gs, np.float32), tile,
                                      np.ascontiguousarray(b_codes, np.uint8),
                                      np.ascontiguousarray(b_scales, np.uint8),
                                      np.ascontiguousarray(b_gscale, np.float32),
                                      np.ascontiguousarray(offsets, np.int32), G, n, kh * 2, out,
                                      _ptr(bound)), "single_pass_gemm")
    return (out, bound) if with_bound else out


def moe_forward_single_pass(x_bf16, topk_idx, topk_prob, num_experts, inter, w1, w2, tile: int,
                            align: int = 1, stage_times: bool = False):
    """Whole expert layer with O12 (online quantize + single-pass FC2) in
    place of the two-pass requantize and FC2.  Returns (y, intermediates
    [, stage seconds]); intermediates["gs_tiles"] holds the per-tile scales."""
    x = np.ascontiguousarray(x_bf16, np.uint16)
    idx = np.ascontiguousarray(topk_idx, np.int32)
    prob = np.ascontiguousarray(topk_prob, np.float32)
    T, H = x.shape
    k = idx.shape[1]
    I = inter
    cap = rows_capacity(T, k, num_experts, align)
    b = dict(
        a1_codes=np.zeros((cap, H // 2), np.uint8), a1_scales=np.zeros((cap, H // 16), np.uint8),
        a1_gscale=np.zeros(cap, np.float32), c_fc1=np.zeros((cap, 2 * I), np.float32),
        d=np.zeros((cap, I), np.uint16), amax_d=np.zeros(cap, np.float32),
        a2_codes=np.zeros((cap, I // 2), np.uint8), a2_scales=np.zeros((cap, I // 16), np.uint8),
        a2_gscale=np.zeros(cap, np.float32), y_rows=np.zeros((cap, H), np.float32),
        offsets=np.zeros(num_experts + 1, np.int32), dst_row=np.zeros((T, k), np.int32),
        row_src=np.zeros(cap, np.int32), row_prob=np.zeros(cap, np.float32))
    st = _MoeBuffers(**{n: b[n].ctypes.data for n in b})
    gs = np.zeros((cap, num_tiles(I, tile)), np.float32)
    y = np.zeros((T, H), np.uint16)
    secs = np.zeros(6, np.float64)
    w1c, w1s, w1g = (np.ascontiguousarray(a) for a in w1)
    w2c, w2s, w2g = (np.ascontiguousarray(a) for a in w2)
    _check(lib().orc_moe_forward_single_pass(
        x, T, H, I, idx, prob, k, num_experts, align, tile,
        w1c.astype(np.uint8, copy=False), w1s.astype(np.uint8, copy=False),
        w1g.astype(np.float32, copy=False), w2c.astype(np.uint8, copy=False),
        w2s.astype(np.uint8, copy=False), w2g.astype(np.float32, copy=False),
        C.byref(st), gs, y, secs.ctypes.data_as(C.c_void_p)), "moe_forward_single_pass")
    b["gs_tiles"] = gs
    if stage_times:
        return y, b, secs
    return y, b

