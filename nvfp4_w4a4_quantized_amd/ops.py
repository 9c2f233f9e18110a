"""Python entry points with the names of the C ABI (include/nvfp4moe.h).

Each function validates tensor devices/dtypes, allocates the outputs with
torch on the input's device, and calls the library on the current stream.
bf16 activations may be passed as torch.bfloat16 or as int16/uint16 bit
patterns; codes and scales are uint8, outer scales float32, indices int32.
"""
from __future__ import annotations

import ctypes as C

import torch

from ._lib import (BackwardIntermediates, Intermediates, NvFp4Error, SinglePassIntermediates,
                   Weights, check, lib, ptr, stream_handle)

__all__ = ["nvfp4_quantize", "moe_rows_capacity", "moe_permute", "moe_permute_noalloc",
           "w4a4_grouped_gemm",
           "w4a4_grouped_gemm_swiglu", "moe_combine", "moe_expert_forward",
           "moe_expert_forward_workspace_size", "moe_expert_forward_single_pass",
           "moe_expert_forward_single_pass_workspace_size", "moe_expert_backward",
           "moe_expert_backward_workspace_size", "SINGLE_PASS_TILE", "NvFp4Weights",
           "StageTimer", "BackwardTimer"]

SINGLE_PASS_TILE = 256   # intermediate columns per online-scale tile of the single-pass layer

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _need(t, dtypes, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise NvFp4Error(f"{name} must be a device tensor (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class NvFp4Weights:
    """NVFP4 expert weights: codes [G, N, K/2] u8, scales [G, N, K/16] u8,
    gscale [G] f32 (one outer scale per expert matrix).  layout 0 is
    row-major; layout 1 holds the same bytes in the grouped GEMM's tiled
    order (nvfp4_pack_weights), the tensor shapes unchanged."""

    def __init__(self, codes, scales, gscale, layout: int = 0):
        self.codes, self.scales, self.gscale = codes, scales, gscale
        self.layout = layout

    def packed(self) -> "NvFp4Weights":
        """The tiled copy of row-major weights (static weights: done once)."""
        if self.layout != 0:
            raise ValueError("weights are already in the tiled layout")
        G, N, kh = self.codes.shape
        pc = torch.empty_like(self.codes)
        ps = torch.empty_like(self.scales)
        check(lib().nvfp4_pack_weights(ptr(self.codes), ptr(self.scales), G, N, kh * 2, ptr(pc),
                                       ptr(ps), stream_handle()), "nvfp4_pack_weights")
        return NvFp4Weights(pc, ps, self.gscale, layout=1)

    @classmethod
    def quantize(cls, w_bf16: torch.Tensor, block_rule: int = 0,
                 blocks_2d: bool = False) -> "NvFp4Weights":
        """Quantizes bf16 weights [G, N, K] with one outer scale per expert
        (block_rule: see nvfp4_quantize; blocks_2d: 16x16 blocks, N % 16 == 0)."""
        G, N, K = w_bf16.shape
        offs = (torch.arange(G + 1, dtype=torch.int32, device=w_bf16.device) * N)
        codes, scales, gscale = nvfp4_quantize(w_bf16.reshape(G * N, K),
                                               scale_domain=2 if blocks_2d else 1,
                                               block_rule=block_rule,
                                               group_offsets=offs)
        return cls(codes.view(G, N, K // 2), scales.view(G, N, K // 16), gscale)

    def c_struct(self) -> Weights:
        return Weights(self.codes.data_ptr(), self.scales.data_ptr(), self.gscale.data_ptr(),
                       self.layout)


def nvfp4_quantize(x, scale_domain: int = 0, group_offsets=None, amax_in=None,
                   block_rule: int = 0, out=None):
    """NVFP4 quantization of a bf16 [rows, k] matrix.  Returns (codes, scales,
    global_scales) with global_scales per row (domain 0) or per group (1).
    block_rule 0: every block maximum maps to 6; 1 / 2: Four-Over-Six with the
    block error measured as a sum of squares / of absolute values.  `out` may
    supply the three output tensors (contiguous, of those shapes)."""
    _need(x, _BF16_LIKE, "x")
    rows, k = x.shape
    dev = x.device
    ng = 0
    if scale_domain in (1, 2):
        _need(group_offsets, (torch.int32,), "group_offsets")
        ng = group_offsets.numel() - 1
    shapes = ((rows, k // 2), (rows, k // 16), (ng if scale_domain in (1, 2) else rows,))
    if out is None:
        codes = torch.empty(shapes[0], dtype=torch.uint8, device=dev)
        scales = torch.empty(shapes[1], dtype=torch.uint8, device=dev)
        gs = torch.empty(shapes[2], dtype=torch.float32, device=dev)
    else:
        codes, scales, gs = out
        for t, n, d, shp in ((codes, "codes", torch.uint8, shapes[0]),
                             (scales, "scales", torch.uint8, shapes[1]),
                             (gs, "global_scales", torch.float32, shapes[2])):
            _need(t, (d,), n)
            if tuple(t.shape) != shp:
                raise ValueError(f"{n}: shape {tuple(t.shape)}, expected {shp}")
    if amax_in is not None:
        _need(amax_in, (torch.float32,), "amax_in")
    check(lib().nvfp4_quantize(ptr(x), rows, k, k, scale_domain, ptr(group_offsets), ng,
                               ptr(amax_in), block_rule, ptr(codes), ptr(scales), ptr(gs),
                               stream_handle()),
          "nvfp4_quantize")
    return codes, scales, gs


def moe_rows_capacity(tokens: int, topk: int, num_experts: int, align: int = 1) -> int:
    return int(lib().moe_rows_capacity(tokens, topk, num_experts, align))


def moe_permute(x, topk_idx, topk_prob, num_experts: int, align: int = 1, block_rule: int = 0,
                workspace=None, library=None):
    """Routing metadata + per-token quantize-scatter.  x may be None (metadata
    only).  Returns a dict of device tensors.  `workspace`: a uint8 device
    tensor of at least moe_permute_workspace_size bytes (allocated here when
    None); `library`: the loaded library to call (the release build by
    default, _lib.debug_lib() for the precondition-checking build)."""
    L = library if library is not None else lib()
    _need(topk_idx, (torch.int32,), "topk_idx")
    _need(topk_prob, (torch.float32,), "topk_prob")
    T, k = topk_idx.shape
    dev = topk_idx.device
    cap = moe_rows_capacity(T, k, num_experts, align)
    out = dict(
        offsets=torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
        dst_row=torch.empty((T, k), dtype=torch.int32, device=dev),
        row_src=torch.empty(cap, dtype=torch.int32, device=dev),
        row_prob=torch.empty(cap, dtype=torch.float32, device=dev))
    H = 0
    if x is not None:
        _need(x, _BF16_LIKE, "x")
        H = x.shape[1]
        out["codes"] = torch.empty((cap, H // 2), dtype=torch.uint8, device=dev)
        out["scales"] = torch.empty((cap, H // 16), dtype=torch.uint8, device=dev)
        out["gscale"] = torch.empty(cap, dtype=torch.float32, device=dev)
    wsb = int(L.moe_permute_workspace_size(T, k, num_experts))
    ws = workspace if workspace is not None else torch.empty(max(wsb, 256), dtype=torch.uint8,
                                                             device=dev)
    _need(ws, (torch.uint8,), "workspace")
    check(L.moe_permute(ptr(x), T, H, ptr(topk_idx), ptr(topk_prob), k, num_experts, align,
                            block_rule, ptr(out["offsets"]), ptr(out["dst_row"]), ptr(out["row_src"]),
                            ptr(out["row_prob"]), ptr(out.get("codes")), ptr(out.get("scales")),
                            ptr(out.get("gscale")), ptr(ws), ws.numel(), stream_handle()),
          "moe_permute")
    return out


def moe_permute_noalloc(x, topk_idx, topk_prob, num_experts: int, align: int = 1,
                        block_rule: int = 0, out=None):
    """moe_permute through the entry point that allocates nothing: the routing
    scratch is the library's static device array.  `out`: a dict of output
    tensors shaped as moe_permute returns them (allocated here when None;
    the library call itself allocates nothing).  Returns that dict."""
    _need(topk_idx, (torch.int32,), "topk_idx")
    _need(topk_prob, (torch.float32,), "topk_prob")
    T, k = topk_idx.shape
    dev = topk_idx.device
    cap = moe_rows_capacity(T, k, num_experts, align)
    H = 0
    if x is not None:
        _need(x, _BF16_LIKE, "x")
        H = x.shape[1]
    if out is None:
        out = dict(
            offsets=torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
            dst_row=torch.empty((T, k), dtype=torch.int32, device=dev),
            row_src=torch.empty(cap, dtype=torch.int32, device=dev),
            row_prob=torch.empty(cap, dtype=torch.float32, device=dev))
        if x is not None:
            out["codes"] = torch.empty((cap, H // 2), dtype=torch.uint8, device=dev)
            out["scales"] = torch.empty((cap, H // 16), dtype=torch.uint8, device=dev)
            out["gscale"] = torch.empty(cap, dtype=torch.float32, device=dev)
    check(lib().moe_permute_noalloc(ptr(x), T, H, ptr(topk_idx), ptr(topk_prob), k, num_experts,
                                    align, block_rule, ptr(out["offsets"]), ptr(out["dst_row"]),
                                    ptr(out["row_src"]), ptr(out["row_prob"]),
                                    ptr(out.get("codes")), ptr(out.get("scales")),
                                    ptr(out.get("gscale")), stream_handle()),
          "moe_permute_noalloc")
    return out


def _gemm_common(a_codes, a_scales, a_gscale, b, group_offsets):
    for t, n, d in ((a_codes, "a_codes", (torch.uint8,)), (a_scales, "a_scales", (torch.uint8,)),
                    (a_gscale, "a_gscale", (torch.float32,)), (b.codes, "b_codes", (torch.uint8,)),
                    (b.scales, "b_scales", (torch.uint8,)), (b.gscale, "b_gscale", (torch.float32,)),
                    (group_offsets, "group_offsets", (torch.int32,))):
        _need(t, d, n)
    G, N, kh = b.codes.shape
    return a_codes.shape[0], G, N, kh * 2


def w4a4_grouped_gemm(a_codes, a_scales, a_gscale, b: NvFp4Weights, group_offsets,
                      out_dtype=torch.float32, out=None):
    rows_cap, G, N, K = _gemm_common(a_codes, a_scales, a_gscale, b, group_offsets)
    code = 0 if out_dtype == torch.float32 else 1
    if out is None:
        out = torch.empty((rows_cap, N), dtype=out_dtype, device=a_codes.device)
    else:
        _need(out, (out_dtype,), "out")
        if tuple(out.shape) != (rows_cap, N):
            raise ValueError(f"out: shape {tuple(out.shape)}, expected {(rows_cap, N)}")
    check(lib().w4a4_grouped_gemm(ptr(a_codes), ptr(a_scales), ptr(a_gscale), rows_cap,
                                  ptr(b.codes), ptr(b.scales), ptr(b.gscale), ptr(group_offsets),
                                  G, N, K, b.layout, code, ptr(out), stream_handle()),
          "w4a4_grouped_gemm")
    return out


def w4a4_grouped_gemm_swiglu(a_codes, a_scales, a_gscale, b: NvFp4Weights, group_offsets,
                             row_prob, with_c: bool = False):
    """FC1 with the weighted SwiGLU epilogue.  Returns (D bf16 [cap, I],
    amax f32 [cap], C f32 [cap, 2I] or None)."""
    rows_cap, G, N2, K = _gemm_common(a_codes, a_scales, a_gscale, b, group_offsets)
    _need(row_prob, (torch.float32,), "row_prob")
    inter = N2 // 2
    dev = a_codes.device
    d = torch.empty((rows_cap, inter), dtype=torch.bfloat16, device=dev)
    amax = torch.zeros(rows_cap, dtype=torch.float32, device=dev)
    c = torch.empty((rows_cap, N2), dtype=torch.float32, device=dev) if with_c else None
    check(lib().w4a4_grouped_gemm_swiglu(ptr(a_codes), ptr(a_scales), ptr(a_gscale), rows_cap,
                                         ptr(b.codes), ptr(b.scales), ptr(b.gscale),
                                         ptr(group_offsets), G, inter, K, b.layout,
                                         ptr(row_prob), ptr(d),
                                         ptr(amax), ptr(c), stream_handle()),
          "w4a4_grouped_gemm_swiglu")
    return d, amax, c


def moe_combine(y_rows, dst_row):
    _need(y_rows, (torch.float32, torch.bfloat16), "y_rows")
    _need(dst_row, (torch.int32,), "dst_row")
    T, k = dst_row.shape
    H = y_rows.shape[1]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=y_rows.device)
    check(lib().moe_combine(ptr(y_rows), 0 if y_rows.dtype == torch.float32 else 1, ptr(dst_row),
                            T, k, H, ptr(y), stream_handle()), "moe_combine")
    return y


def moe_expert_forward_workspace_size(tokens, hidden, inter, topk, num_experts, align=1) -> int:
    return int(lib().moe_expert_forward_workspace_size(tokens, hidden, inter, topk, num_experts,
                                                       align))


class StageTimer:
    """Six HIP events recorded by moe_expert_forward at its stage boundaries:
    route+quantize, FC1+SwiGLU, requantize, FC2, combine."""

    NAMES = ("route_quantize", "fc1_swiglu", "requantize", "fc2", "combine")

    def __init__(self):
        L = lib()
        self.events = (C.c_void_p * 6)()
        for i in range(6):
            h = C.c_void_p()
            check(L.nvfp4_event_create(C.byref(h)), "nvfp4_event_create")
            self.events[i] = h.value

    def elapsed_ms(self):
        out = {}
        ms = C.c_float()
        for i, n in enumerate(self.NAMES):
            check(lib().nvfp4_event_elapsed_ms(self.events[i], self.events[i + 1], C.byref(ms)),
                  "nvfp4_event_elapsed_ms")
            out[n] = ms.value
        return out

    def close(self):
        for i in range(6):
            if self.events[i]:
                lib().nvfp4_event_destroy(self.events[i])
                self.events[i] = None


def moe_expert_forward(x, topk_idx, topk_prob, num_experts: int, inter: int,
                       w1: NvFp4Weights, w2: NvFp4Weights, align: int = 1, workspace=None,
                       debug: bool = False, fc1_out: bool = False, y_rows_f32: bool = False,
                       timer: StageTimer | None = None, y=None, act_block_rule: int = 0,
                       act_scale_domain: int = 0, library=None):
    """The whole expert layer.  Returns y (bf16 [T, H]); with debug=True also a
    dict of the intermediates (allocated here, written by the library).
    act_scale_domain: 0 one activation outer scale per token, 1 per tensor.
    `library`: the loaded library to call (release build by default)."""
    L = library if library is not None else lib()
    _need(x, _BF16_LIKE, "x")
    _need(topk_idx, (torch.int32,), "topk_idx")
    _need(topk_prob, (torch.float32,), "topk_prob")
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    wsb = int(L.moe_expert_forward_workspace_size(T, H, inter, k, num_experts, align))
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dbg = None
    inter_t = None
    if debug:
        cap = moe_rows_capacity(T, k, num_experts, align)
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
        inter_t = dict(
            expert_offsets=e(num_experts + 1, torch.int32), dst_row=e((T, k), torch.int32),
            row_src=e(cap, torch.int32), row_prob=e(cap, torch.float32),
            a1_codes=e((cap, H // 2), torch.uint8), a1_scales=e((cap, H // 16), torch.uint8),
            a1_gscale=e(cap, torch.float32), d=e((cap, inter), torch.bfloat16),
            amax_d=e(cap, torch.float32), a2_codes=e((cap, inter // 2), torch.uint8),
            a2_scales=e((cap, inter // 16), torch.uint8), a2_gscale=e(cap, torch.float32),
            y_rows=e((cap, H), torch.bfloat16))
        if fc1_out:
            inter_t["fc1_out"] = e((cap, 2 * inter), torch.float32)
        if y_rows_f32:
            inter_t["y_rows_f32"] = e((cap, H), torch.float32)
        dbg = Intermediates(**{n: t.data_ptr() for n, t in inter_t.items()})
    ev = timer.events if timer is not None else None
    check(L.moe_expert_forward(ptr(x), T, H, inter, ptr(topk_idx), ptr(topk_prob), k,
                                   num_experts, align, act_block_rule, act_scale_domain,
                                   C.byref(w1.c_struct()),
                                   C.byref(w2.c_struct()), ptr(y), ptr(workspace),
                                   workspace.numel(), C.byref(dbg) if dbg is not None else None,
                                   C.cast(ev, C.c_void_p) if ev is not None else None,
                                   stream_handle()), "moe_expert_forward")
    if debug:
        return y, inter_t
    return y


class SinglePassTimer(StageTimer):
    """Four HIP events recorded by moe_expert_forward_single_pass: routing +
    quantize, the fused FC1 -> SwiGLU -> quantize -> FC2 kernel, combine."""

    NAMES = ("route_quantize", "fused_fc1_fc2", "combine")

    def __init__(self):
        L = lib()
        self.events = (C.c_void_p * 4)()
        for i in range(4):
            h = C.c_void_p()
            check(L.nvfp4_event_create(C.byref(h)), "nvfp4_event_create")
            self.events[i] = h.value

    def close(self):
        for i in range(4):
            if self.events[i]:
                lib().nvfp4_event_destroy(self.events[i])
                self.events[i] = None


def moe_expert_forward_single_pass_workspace_size(tokens, hidden, inter, topk, num_experts,
                                                  align=1) -> int:
    return int(lib().moe_expert_forward_single_pass_workspace_size(tokens, hidden, inter, topk,
                                                                   num_experts, align))


def moe_expert_forward_single_pass(x, topk_idx, topk_prob, num_experts: int, inter: int,
                                   w1: NvFp4Weights, w2: NvFp4Weights, align: int = 1,
                                   workspace=None, debug: bool = False, fc1_out: bool = False,
                                   y_rows_f32: bool = False, timer=None, y=None):
    """The expert layer with the single-pass FC1 -> SwiGLU -> quantize -> FC2
    kernel (online amax compensation, tiles of SINGLE_PASS_TILE columns).
    Returns y (bf16 [T, H]); with debug=True also a dict of the intermediates:
    routing maps, a1 rows, fc1_out (if asked), p (bf16 weighted SwiGLU),
    a2_codes / a2_scales (the online quantization), gs_tiles, y_rows (bf16, or
    y_rows_f32 if asked)."""
    _need(x, _BF16_LIKE, "x")
    _need(topk_idx, (torch.int32,), "topk_idx")
    _need(topk_prob, (torch.float32,), "topk_prob")
    T, H = x.shape
    k = topk_idx.shape[1]
    dev = x.device
    wsb = moe_expert_forward_single_pass_workspace_size(T, H, inter, k, num_experts, align)
    if workspace is None:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=dev)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dbg = None
    inter_t = None
    if debug:
        cap = moe_rows_capacity(T, k, num_experts, align)
        nt = (inter + SINGLE_PASS_TILE - 1) // SINGLE_PASS_TILE
        e = lambda shape, dt: torch.zeros(shape, dtype=dt, device=dev)  # noqa: E731
        inter_t = dict(
            expert_offsets=e(num_experts + 1, torch.int32), dst_row=e((T, k), torch.int32),
            row_src=e(cap, torch.int32), row_prob=e(cap, torch.float32),
            a1_codes=e((cap, H // 2), torch.uint8), a1_scales=e((cap, H // 16), torch.uint8),
            a1_gscale=e(cap, torch.float32), p=e((cap, inter), torch.bfloat16),
            a2_codes=e((cap, inter // 2), torch.uint8), a2_scales=e((cap, inter // 16), torch.uint8),
            gs_tiles=e((cap, nt), torch.float32), y_rows=e((cap, H), torch.bfloat16))
        if fc1_out:
            inter_t["fc1_out"] = e((cap, 2 * inter), torch.float32)
        if y_rows_f32:
            inter_t["y_rows_f32"] = e((cap, H), torch.float32)
        dbg = SinglePassIntermediates(**{n: t.data_ptr() for n, t in inter_t.items()})
    ev = timer.events if timer is not None else None
    check(lib().moe_expert_forward_single_pass(
        ptr(x), T, H, inter, ptr(topk_idx), ptr(topk_prob), k, num_experts, align,
        C.byref(w1.c_struct()), C.byref(w2.c_struct()), ptr(y), ptr(workspace), workspace.numel(),
        C.byref(dbg) if dbg is not None else None,
        C.cast(ev, C.c_void_p) if ev is not None else None, stream_handle()),
        "moe_expert_forward_single_pass")
    if debug:
        return y, inter_t
    return y



class BackwardTimer(StageTimer):
    """Eight HIP events recorded by moe_expert_backward around its stages, in
    the order they run: the dgrad tile tables, FC2 dgrad, the SwiGLU
    backward, FC1 dgrad, the dx / dprob reductions, FC2 wgrad, FC1 wgrad."""

    NAMES = ("tables", "fc2_dgrad", "swiglu_bwd", "fc1_dgrad", "reduce", "fc2_wgrad",
             "fc1_wgrad")

    def __init__(self):
        L = lib()
        self.events = (C.c_void_p * 8)()
        for i in range(8):
            h = C.c_void_p()
            check(L.nvfp4_event_create(C.byref(h)), "nvfp4_event_create")
            self.events[i] = h.value

    def close(self):
        for i in range(8):
            if self.events[i]:
                lib().nvfp4_event_destroy(self.events[i])
                self.events[i] = None


def moe_expert_backward_workspace_size(rows_cap, hidden, inter, num_experts) -> int:
    return int(lib().moe_expert_backward_workspace_size(rows_cap, hidden, inter, num_experts))


def moe_expert_backward(dy, x, fc1_out, d, expert_offsets, row_src, row_prob, dst_row,
                        w1, w2, workspace=None, debug: bool = False,
                        dx_rows_f32: bool = False, timer: BackwardTimer | None = None,
                        out=None):
    """Gradients of the expert layer (straight-through, BF16 GEMMs).
    dy, x: bf16 [T, H]; fc1_out: fp32 [cap, 2I] and d: bf16 [cap, I], the
    forward's FC1 output and FC2 input; the forward's routing arrays; w1 bf16
    [E, 2I, H], w2 bf16 [E, H, I].  Returns dict(dx, dw1, dw2, dprob); with
    debug=True a second dict of the intermediates (dd, dc, dp_rows, dx_rows,
    and dx_rows_f32 if asked).  `out`: optional dict of preallocated outputs
    with those four names."""
    for t, n in ((dy, "dy"), (x, "x"), (d, "d"), (w1, "w1"), (w2, "w2")):
        _need(t, _BF16_LIKE, n)
    _need(fc1_out, (torch.float32,), "fc1_out")
    _need(row_prob, (torch.float32,), "row_prob")
    for t, n in ((expert_offsets, "expert_offsets"), (row_src, "row_src"), (dst_row, "dst_row")):
        _need(t, (torch.int32,), n)
    T, H = dy.shape
    E = w1.shape[0]
    inter = w2.shape[2]
    k = dst_row.shape[1]
    cap = d.shape[0]
    if (tuple(x.shape) != (T, H) or tuple(fc1_out.shape) != (cap, 2 * inter)
            or tuple(d.shape) != (cap, inter) or tuple(w1.shape) != (E, 2 * inter, H)
            or tuple(w2.shape) != (E, H, inter) or expert_offsets.numel() != E + 1
            or row_src.numel() < cap or row_prob.numel() < cap or dst_row.shape[0] != T):
        raise NvFp4Error("moe_expert_backward: inconsistent shapes")
    dev = dy.device
    L = lib()
    wsb = int(L.moe_expert_backward_workspace_size(cap, H, inter, E))
    if workspace is None:
        workspace = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = dict(dx=torch.empty((T, H), dtype=torch.bfloat16, device=dev),
                   dw1=torch.empty((E, 2 * inter, H), dtype=torch.float32, device=dev),
                   dw2=torch.empty((E, H, inter), dtype=torch.float32, device=dev),
                   dprob=torch.empty((T, k), dtype=torch.float32, device=dev))
    dbg = None
    inter_t = None
    if debug:
        e = lambda shape, dt: torch.empty(shape, dtype=dt, device=dev)  # noqa: E731
        inter_t = dict(dd=e((cap, inter), torch.bfloat16), dc=e((cap, 2 * inter), torch.bfloat16),
                       dp_rows=e(cap, torch.float32), dx_rows=e((cap, H), torch.bfloat16))
        if dx_rows_f32:
            inter_t["dx_rows_f32"] = e((cap, H), torch.float32)
        dbg = BackwardIntermediates(**{n: t.data_ptr() for n, t in inter_t.items()})
    ev = timer.events if timer is not None else None
    check(L.moe_expert_backward(ptr(dy), ptr(x), T, H, inter, k, E, cap, ptr(fc1_out), ptr(d),
                                ptr(expert_offsets), ptr(row_src), ptr(row_prob), ptr(dst_row),
                                ptr(w1), ptr(w2), ptr(out["dx"]), ptr(out["dw1"]),
                                ptr(out["dw2"]), ptr(out["dprob"]), ptr(workspace),
                                workspace.numel(), C.byref(dbg) if dbg is not None else None,
                                C.cast(ev, C.c_void_p) if ev is not None else None,
                                stream_handle()), "moe_expert_backward")
    if debug:
        return out, inter_t
    return out
