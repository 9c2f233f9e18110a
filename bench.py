"""Benchmark of the NVFP4 W4A4 MoE expert layer on one MI355X.

One step = one moe_expert_forward call: routing metadata + per-token NVFP4
quantize-permute, FC1 grouped GEMM with the weighted SwiGLU + row-amax
epilogue, requantization of D, FC2 grouped GEMM, combine.  Weights are
quantized once before timing and stored in the grouped GEMM's tiled layout
(static weights).  Inputs are seeded synthetic
tensors with the shapes of the Qwen3-30B-A3B expert layer (T=8192 tokens,
hidden 2048, 128 experts, top-8, intermediate 768, Zipf(1.1)-biased router),
resident in HBM before the timed region.

Prints one JSON line (rank 0):
  value        tokens/s of the whole layer, timed over uninstrumented steps
  stage_ms     per-stage averages from HIP events recorded on the launch
               stream between the stages, over the same number of further
               steps (each event idles the GPU a few microseconds, so these
               steps are not the ones the headline times)
  roofline     the FC1 kernel (dominant): algorithmic FLOPs per launch over its
               average duration from those events
  cpu_baseline the CPU oracle timed on a bounded token sample of the workload
  four_over_six the same layer with Four-Over-Six (MSE) weights and activations
               (a secondary line; the headline is the standard block rule)
  single_pass  the same layer with FC1 -> SwiGLU -> quantize -> FC2 fused by
               online amax compensation
  backward     the layer's backward (straight-through, BF16 GEMMs on the saved
               bf16 operands): tokens/s, per-GEMM TFLOP/s and bf16-peak fraction
  secondary    the other measured shapes, each timed the same way:
               dense_t8192   W4A4 attention projections (per-token quantize +
                             G=1 GEMM for QKV, then for O-proj), tokens/s and
                             fraction of the dense fp16 MFMA peak
               decode_t256   the expert layer at 256 tokens with uniform routing,
                             bound by streaming the weights: fraction of HBM peak
                             (three weight copies rotated, 1 GB, so that the
                             256 MB last-level cache cannot hold them)
               long_t32768   the expert layer at 32768 tokens, Student-t(3)
                             activations with outlier channels and zero rows,
                             Zipf(1.3) routing
               The expert layers reuse the headline's quantized weights (same
               shapes and N(0, 0.02) distribution; the timing does not depend on
               weight values).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_F16_TFLOPS = 2500.0      # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="qwen3_30b_a3b_moe_t8192")
    p.add_argument("--cpu-tokens", type=int, default=4096,
                   help="tokens of the oracle's CPU-baseline sample (0 = skip)")
    p.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "fc1_traffic.json"),
                   help="JSON record of measured HBM bytes per FC1 launch (rocprof PMC); "
                        "ignored when the GEMM source changed since it was taken")
    p.add_argument("--four-over-six", type=int, default=1,
                   help="also time the layer with Four-Over-Six (MSE) weights and activations and "
                        "report it under 'four_over_six' (0 = skip); the headline stays the "
                        "standard rule")
    p.add_argument("--single-pass", type=int, default=1,
                   help="also time the layer with the single-pass FC1 -> SwiGLU -> quantize -> FC2 "
                        "kernel (online amax compensation) and report it under 'single_pass' "
                        "(0 = skip)")
    p.add_argument("--backward", type=int, default=1,
                   help="also time the expert layer's backward (moe_expert_backward) on the "
                        "headline workload (0: skip)")
    p.add_argument("--secondary", default="dense,decode,long",
                   help="comma list of the secondary workloads to time and report under "
                        "'secondary' (dense: the attention projections; decode: the 256-token "
                        "layer; long: the 32768-token layer); empty or 0 = none")
    p.add_argument("--skip-headline", action="store_true",
                   help="profiling aid: quantize the headline workload's weights but time only "
                        "the secondary workloads (the headline fields are then null)")
    p.add_argument("--settle-max-steps", type=int, default=400,
                   help="most extra untimed steps of the clock-settling phase (0: none, for "
                        "profiler runs where only the kernels' own figures are used)")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="after timing, run plain device copies of this many MiB (a known-size "
                        "kernel for scaling the rocprof FETCH_SIZE/WRITE_SIZE counters)")
    return p.parse_args()


def moe_algorithmic(w):
    """FC1 and FC2 flops and the bytes of moe_permute's quantize + permute:
    read x and the routing, write each routed row (codes, scales, s_g) and
    the maps (row_src, row_prob per row; dst_row per entry)."""
    R = w.routed_rows
    H, I, T, k = w.hidden, w.inter, w.tokens, w.topk
    fc1 = 2.0 * R * 2 * I * H
    fc2 = 2.0 * R * H * I
    qbytes = T * H * 2 + T * k * 8 + R * (H // 2 + H // 16 + 4) + R * 8 + T * k * 4
    return fc1, fc2, qbytes


def layer_route_bytes(w):
    """Bytes of the layer's routing stage, which quantizes each token once and
    lets FC1 gather the routed rows: read x and the routing, write each
    token's row (codes, scales, s_g), and per routed row its token, router
    weight and outer scale, per entry its row and chunk rank (one byte,
    written and read)."""
    R, H, T, k = w.routed_rows, w.hidden, w.tokens, w.topk
    return T * H * 2 + T * k * 8 + T * (H // 2 + H // 16 + 4) + R * 12 + T * k * (4 + 2)


def moe_layer_bytes(w):
    """HBM bytes the layer must move with its intermediates in HBM: the
    routing stage's bytes, both weight sets (codes, block scales, outer
    scales) read once, the token rows read by FC1 (once each) with each routed
    row's token, outer scale and router weight, D written and read back, A2
    written and read, the expert rows written by FC2 and read by the combine,
    y written."""
    R, H, I, T, E = w.routed_rows, w.hidden, w.inter, w.tokens, w.experts
    weights = E * 2 * I * (H // 2 + H // 16) + E * H * (I // 2 + I // 16) + 2 * E * 4
    a1 = T * (H // 2 + H // 16) + R * 12          # token rows; row_src, s_g, router weight
    d = 2 * R * I * 2 + 2 * R * 4                 # D bf16 and its row amax, each both ways
    a2 = 2 * R * (I // 2 + I // 16 + 4)
    rows = 2 * R * H * 2
    return layer_route_bytes(w) + weights + a1 + d + a2 + rows + T * H * 2


SETTLE_BATCH = 10            # steps per batch of the clock-settling phase
SETTLE_TOL = 0.01            # stable: a batch within 1% of the previous one
SETTLE = {"max_steps": 400}  # at most this many settling steps (--settle-max-steps)

SETTLE_LOG = {}


def settle_clocks(step, label):
    """The GPU raises its clocks over the first few hundred milliseconds of
    sustained work (right after a short warm-up the layer's step time falls
    from about 0.90 to 0.70 ms over 20 steps, and again after 2 s idle).
    After the requested warm-up, steps run in batches of SETTLE_BATCH, each
    timed by a pair of events, until one batch is within SETTLE_TOL of the
    previous one (at most SETTLE_MAX_STEPS steps).  The extra steps are
    reported in the output line ('clock_settle'), never hidden."""
    import torch
    batches = []
    n = 0
    while n < SETTLE["max_steps"]:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(SETTLE_BATCH):
            step(None)
        e1.record()
        torch.cuda.synchronize()
        n += SETTLE_BATCH
        batches.append(e0.elapsed_time(e1) / SETTLE_BATCH)
        if len(batches) >= 2 and abs(batches[-1] - batches[-2]) <= SETTLE_TOL * batches[-2]:
            break
    SETTLE_LOG[label] = {"extra_steps": n, "batch_ms_per_step": [round(b, 4) for b in batches]}
    log(f"clock settle ({label}): {n} extra steps, ms/step per batch "
        + ", ".join(f"{b:.4f}" for b in batches))


def run_steps(step, steps, warmup, label, timer_cls=None):
    """Warm-up, clock settling (settle_clocks), then `steps` uninstrumented
    calls timed by the host clock around device synchronisations; with
    timer_cls, the same number of steps again with a fresh timer per step,
    whose per-stage averages are returned."""
    import torch
    log(f"warmup {warmup} ({label})")
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    settle_clocks(step, label)
    log(f"timing {steps} steps ({label})")
    t0 = time.perf_counter()
    for _ in range(steps):
        step(None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = None
    if timer_cls is not None:
        timers = [timer_cls() for _ in range(steps)]
        log(f"stage events over {steps} more steps ({label})")
        for i in range(steps):
            step(timers[i])
        torch.cuda.synchronize()
        stages = {n: float(np.mean([t.elapsed_ms()[n] for t in timers])) for n in timer_cls.NAMES}
        for t in timers:
            t.close()
    return wall, stages


def bench_permute(args, w, x, idx, prob, qbytes):
    """moe_permute on the headline routing: the quantize + permute entry point
    that writes the k routed copies of every token (the permuted layout).
    Warm-up, clock settling, then `steps` calls between two events."""
    import torch

    from nvfp4_w4a4_quantized_amd import _lib, ops
    L = ops.lib()
    ws = torch.empty(int(L.moe_permute_workspace_size(w.tokens, w.topk, w.experts)),
                     dtype=torch.uint8, device=x.device)
    out = ops.moe_permute(x, idx, prob, w.experts, workspace=ws)   # allocates the outputs once
    p = _lib.ptr
    args_c = (p(x), w.tokens, w.hidden, p(idx), p(prob), w.topk, w.experts, 1, 0,
              p(out["offsets"]), p(out["dst_row"]), p(out["row_src"]), p(out["row_prob"]),
              p(out["codes"]), p(out["scales"]), p(out["gscale"]), p(ws), ws.numel(),
              _lib.stream_handle())

    def step(_):
        _lib.check(L.moe_permute(*args_c), "moe_permute")
    for _ in range(args.warmup):
        step(None)
    settle_clocks(step, "moe_permute")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step(None)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    del out, ws
    return {"ms": ms, "bytes": qbytes, "gbps": qbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": qbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "note": "moe_permute (routing + per-token quantize + the k routed copies), timed "
                    "between two events over the steps, outputs allocated once"}


def bench_single_pass(args, w, x, idx, prob, W1, W2):
    """The headline layer with FC1 -> SwiGLU -> quantize -> FC2 fused by online
    amax compensation (one kernel per 128-row block; the intermediate and its
    quantization stay on chip).  Timed like the headline."""
    import torch

    from nvfp4_w4a4_quantized_amd.ops import (SinglePassTimer, moe_expert_forward_single_pass,
                                              moe_expert_forward_single_pass_workspace_size)
    log("single-pass FC1 -> FC2 (online amax compensation)")
    ws = torch.empty(moe_expert_forward_single_pass_workspace_size(w.tokens, w.hidden, w.inter,
                                                                    w.topk, w.experts),
                     dtype=torch.uint8, device=x.device)
    y = torch.empty((w.tokens, w.hidden), dtype=torch.bfloat16, device=x.device)
    torch.cuda.synchronize()

    def step(timer):
        moe_expert_forward_single_pass(x, idx, prob, w.experts, w.inter, W1, W2, workspace=ws,
                                       y=y, timer=timer)
    wall, st = run_steps(step, args.steps, args.warmup, "single pass", SinglePassTimer)
    ms = wall * 1e3 / args.steps
    fc1, fc2, _ = moe_algorithmic(w)
    R, I = w.routed_rows, w.inter
    log("stages single pass (ms, HIP events): " + ", ".join(f"{k}={v:.4f}" for k, v in st.items()))
    del ws, y
    return {
        "kernel": "moe_expert_forward_single_pass (tiles of 256 intermediate columns)",
        "value": w.tokens * args.steps / wall, "unit": "tokens/s", "ms_per_step": ms,
        "effective_tflops": (fc1 + fc2) / (ms * 1e-3) / 1e12,
        "frac_of_f16_peak": (fc1 + fc2) / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "stage_ms": st,
        "fused_kernel_tflops": (fc1 + fc2) / (st["fused_fc1_fc2"] * 1e-3) / 1e12,
        "hbm_bytes_not_moved": 2 * R * I * 2 + 2 * R * 4 + 2 * R * (I // 2 + I // 16 + 4),
    }


def bench_backward(args, w, x, idx, prob, W1, W2, bf):
    """The expert layer's backward (straight-through, BF16 GEMMs on the saved
    bf16 operands): the forward runs once with its intermediates to supply
    the routing, FC1's output and FC2's input, then moe_expert_backward is
    timed like the headline.  Algorithmic flops: four GEMMs over the routed
    rows (padding excluded), 2 R H I each for FC2's dgrad and wgrad and
    2 R 2I H each for FC1's."""
    import torch

    from nvfp4_w4a4_quantized_amd.ops import (BackwardTimer, moe_expert_backward,
                                              moe_expert_backward_workspace_size,
                                              moe_expert_forward)
    log("backward: forward once for the saved tensors")
    _, it = moe_expert_forward(x, idx, prob, w.experts, w.inter, W1, W2, debug=True,
                               fc1_out=True)
    from nvfp4_w4a4_quantized_amd.workloads import random_bf16
    dy = bf(random_bf16(np.random.Generator(np.random.PCG64(7)), (w.tokens, w.hidden)))
    w1b, w2b = bf(w.w1), bf(w.w2)
    cap = it["d"].shape[0]
    ws = torch.empty(moe_expert_backward_workspace_size(cap, w.hidden, w.inter, w.experts),
                     dtype=torch.uint8, device=x.device)
    out = dict(dx=torch.empty_like(x),
               dw1=torch.empty((w.experts, 2 * w.inter, w.hidden), dtype=torch.float32,
                               device=x.device),
               dw2=torch.empty((w.experts, w.hidden, w.inter), dtype=torch.float32,
                               device=x.device),
               dprob=torch.empty((w.tokens, w.topk), dtype=torch.float32, device=x.device))
    torch.cuda.synchronize()

    def step(timer):
        moe_expert_backward(dy, x, it["fc1_out"], it["d"], it["expert_offsets"], it["row_src"],
                            it["row_prob"], it["dst_row"], w1b, w2b, workspace=ws, out=out,
                            timer=timer)
    wall, st = run_steps(step, args.steps, args.warmup, "backward", BackwardTimer)
    ms = wall * 1e3 / args.steps
    R, H, I = w.routed_rows, w.hidden, w.inter
    f2 = 2.0 * R * H * I
    f1 = 2.0 * R * 2 * I * H
    gemm = {"fc2_dgrad": f2, "fc2_wgrad": f2, "fc1_dgrad": f1, "fc1_wgrad": f1}
    total = 2 * f1 + 2 * f2
    log("stages backward (ms, HIP events): " + ", ".join(f"{k}={v:.4f}" for k, v in st.items()))
    res = {
        "kernel": "moe_expert_backward (bf16 MFMA, fp32 accumulate; dW fp32, dx bf16)",
        "value": w.tokens * args.steps / wall, "unit": "tokens/s", "ms_per_step": ms,
        "flops": total, "effective_tflops": total / (ms * 1e-3) / 1e12,
        "frac_of_bf16_peak": total / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "stage_ms": st,
        "gemm_tflops": {k: v / (st[k] * 1e-3) / 1e12 for k, v in gemm.items()},
        "gemm_frac_of_bf16_peak": {k: v / (st[k] * 1e-3) / 1e12 / PEAK_F16_TFLOPS
                                   for k, v in gemm.items()},
    }
    del ws, out, it, w1b, w2b, dy
    return res


class _TorchStages:
    """Events recorded on the current stream between the dense path's calls."""
    NAMES = ("quantize_qkv", "gemm_qkv", "quantize_o", "gemm_o")

    def __init__(self):
        import torch
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]

    def mark(self, i):
        self.ev[i].record()

    def elapsed_ms(self):
        return {n: self.ev[i].elapsed_time(self.ev[i + 1]) for i, n in enumerate(self.NAMES)}

    def close(self):
        pass


def bench_dense(args, dev, bf):
    """W4A4 attention projections, 8192 tokens: per-token NVFP4 quantize of the
    input, then one G=1 grouped GEMM with bf16 output, for QKV (K=2048,
    N=5120) and O-proj (K=4096, N=2048) with independent inputs."""
    import torch

    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights, nvfp4_quantize, w4a4_grouped_gemm
    from nvfp4_w4a4_quantized_amd.workloads import make_dense
    log("generating the dense projections workload")
    d = make_dense()
    T = d.tokens
    flops = 0.0
    qbytes = 0
    legs = []
    for name, xb, wb in d.projections:
        N, K = wb.shape
        x = bf(xb)
        W = NvFp4Weights.quantize(bf(wb).view(1, N, K)).packed()
        q = (torch.empty((T, K // 2), dtype=torch.uint8, device=dev),
             torch.empty((T, K // 16), dtype=torch.uint8, device=dev),
             torch.empty(T, dtype=torch.float32, device=dev))
        out = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        offs = torch.tensor([0, T], dtype=torch.int32, device=dev)
        legs.append((x, W, q, out, offs))
        flops += 2.0 * T * N * K
        qbytes += T * K * 2 + T * (K // 2 + K // 16 + 4)
    torch.cuda.synchronize()

    def step(timer):
        for i, (x, W, q, out, offs) in enumerate(legs):
            if timer:
                timer.mark(2 * i)
            nvfp4_quantize(x, out=q)
            if timer:
                timer.mark(2 * i + 1)
            w4a4_grouped_gemm(q[0], q[1], q[2], W, offs, out_dtype=torch.bfloat16, out=out)
        if timer:
            timer.mark(4)

    wall, st = run_steps(step, args.steps, args.warmup, "dense projections", _TorchStages)
    ms = wall * 1e3 / args.steps
    gemm_ms = st["gemm_qkv"] + st["gemm_o"]
    return {
        "workload": d.name, "tokens": T,
        "projections": "qkv K=2048 N=5120, o_proj K=4096 N=2048 (independent inputs)",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
        "flops_per_step": flops,
        "effective_tflops": flops / (ms * 1e-3) / 1e12,
        "frac_of_f16_peak": flops / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "stage_ms": st,
        "gemm_only_tflops": flops / (gemm_ms * 1e-3) / 1e12,
        "gemm_only_frac_of_f16_peak": flops / (gemm_ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "quantize_gbps": qbytes / ((st["quantize_qkv"] + st["quantize_o"]) * 1e-3) / 1e9,
    }


def bench_moe_secondary(args, dev, bf, wid, W1, W2, weight_copies, label):
    """The expert layer on another token count / routing, with the headline's
    weights (rotated over `weight_copies` copies)."""
    import torch

    from nvfp4_w4a4_quantized_amd.ops import (NvFp4Weights, StageTimer, moe_expert_forward,
                                              moe_expert_forward_workspace_size)
    from nvfp4_w4a4_quantized_amd.workloads import make_moe
    log(f"generating workload {label} (routing and activations)")
    w = make_moe(wid, with_weights=False)
    x = bf(w.x)
    idx = torch.from_numpy(w.topk_idx).to(dev)
    prob = torch.from_numpy(w.topk_prob).to(dev)
    sets = [(W1, W2)]
    for _ in range(weight_copies - 1):
        sets.append(tuple(NvFp4Weights(V.codes.clone(), V.scales.clone(), V.gscale.clone(),
                                       V.layout) for V in (W1, W2)))
    ws = torch.empty(moe_expert_forward_workspace_size(w.tokens, w.hidden, w.inter, w.topk,
                                                       w.experts), dtype=torch.uint8, device=dev)
    y = torch.empty((w.tokens, w.hidden), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    it = [0]

    def step(timer):
        V1, V2 = sets[it[0] % len(sets)]
        it[0] += 1
        moe_expert_forward(x, idx, prob, w.experts, w.inter, V1, V2, workspace=ws, y=y,
                           timer=timer)

    wall, st = run_steps(step, args.steps, args.warmup, label, StageTimer)
    ms = wall * 1e3 / args.steps
    fc1, fc2, qbytes = moe_algorithmic(w)
    lbytes = moe_layer_bytes(w)
    rbytes = layer_route_bytes(w)
    rec = {
        "workload": w.name, "tokens": w.tokens, "routed_rows": w.routed_rows,
        "active_experts": w.meta["active_experts"],
        "cv_rows_per_expert": round(w.meta["cv_rows_per_expert"], 3),
        "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
        "effective_tflops": (fc1 + fc2) / (ms * 1e-3) / 1e12,
        "frac_of_f16_peak": (fc1 + fc2) / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "layer_bytes": lbytes,
        "hbm_gbps": lbytes / (ms * 1e-3) / 1e9,
        "frac_of_hbm_peak": lbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "weight_copies_rotated": weight_copies,
        "stage_ms": st,
        "route_quantize_bytes": rbytes,
        "route_quantize_gbps": rbytes / (st["route_quantize"] * 1e-3) / 1e9,
    }
    del ws, y, sets
    return rec


def run_secondary(args, dev, bf, W1, W2):
    names = [n for n in str(args.secondary).replace(" ", "").split(",") if n and n != "0"]
    unknown = set(names) - {"dense", "decode", "long"}
    if unknown:
        raise SystemExit(f"bench.py: unknown secondary workload(s) {sorted(unknown)}")
    sec = {}
    if "dense" in names:
        sec["dense_t8192"] = bench_dense(args, dev, bf)
    if "decode" in names:
        sec["decode_t256"] = bench_moe_secondary(args, dev, bf, "decode_moe_t256", W1, W2, 3,
                                                 "decode_t256")
    if "long" in names:
        sec["long_t32768"] = bench_moe_secondary(args, dev, bf, "long_heavytail_moe_t32768",
                                                 W1, W2, 1, "long_t32768")
    for k, v in sec.items():
        log(f"{k}: {v['value']:.4g} tokens/s, {v['ms_per_step']:.4f} ms/step")
    return sec


STAGE_NAMES = ("route_quantize", "fc1", "swiglu", "requantize", "fc2", "combine")


def _oracle_layer(O, w, W1, W2, n_tokens, threads):
    """One oracle run of the layer on the first n_tokens tokens: wall seconds
    and the oracle's own per-stage seconds (steady clock)."""
    O.set_num_threads(threads)
    t0 = time.perf_counter()
    _, _, secs = O.moe_forward(w.x[:n_tokens], w.topk_idx[:n_tokens], w.topk_prob[:n_tokens],
                               w.experts, w.inter, W1, W2, stage_times=True)
    dt = time.perf_counter() - t0
    return dt, {n: round(float(v), 4) for n, v in zip(STAGE_NAMES, secs)}


def cpu_baseline(w, n_tokens):
    """The CPU oracle, as it stands, on bounded samples (one run each):
      - the headline workload's first n_tokens tokens on all host threads
        (the reported value, with the oracle's per-stage seconds);
      - the 256-token tiny layer, all threads and one thread;
      - the decode-shaped layer (256 tokens, Qwen3 shapes): all 256 tokens on
        all threads and a 32-token sample on one thread.  It uses the
        headline's oracle-quantized weights (same shapes and distribution;
        the oracle's time does not depend on weight values)."""
    from oracle import oracle as O
    from nvfp4_w4a4_quantized_amd.workloads import make_moe
    E, I, H = w.experts, w.inter, w.hidden
    cores = len(os.sched_getaffinity(0))
    log(f"cpu baseline: oracle weight quantization (offline, untimed), {cores} host threads")
    O.set_num_threads(cores)
    ow1 = O.quantize(w.w1.reshape(E * 2 * I, H), domain=1,
                     group_offsets=np.arange(E + 1, dtype=np.int32) * 2 * I)
    ow2 = O.quantize(w.w2.reshape(E * H, I), domain=1,
                     group_offsets=np.arange(E + 1, dtype=np.int32) * H)
    W1 = (ow1[0].reshape(E, 2 * I, H // 2), ow1[1].reshape(E, 2 * I, H // 16), ow1[2])
    W2 = (ow2[0].reshape(E, H, I // 2), ow2[1].reshape(E, H, I // 16), ow2[2])
    dt, stages = _oracle_layer(O, w, W1, W2, n_tokens, cores)
    log(f"cpu baseline: {n_tokens} tokens in {dt:.2f} s on {O.num_threads()} threads; stages {stages}")
    extra = {}
    w0 = make_moe(0)
    E0, I0, H0 = w0.experts, w0.inter, w0.hidden
    q1 = O.quantize(w0.w1.reshape(E0 * 2 * I0, H0), domain=1,
                    group_offsets=np.arange(E0 + 1, dtype=np.int32) * 2 * I0)
    q2 = O.quantize(w0.w2.reshape(E0 * H0, I0), domain=1,
                    group_offsets=np.arange(E0 + 1, dtype=np.int32) * H0)
    V1 = (q1[0].reshape(E0, 2 * I0, H0 // 2), q1[1].reshape(E0, 2 * I0, H0 // 16), q1[2])
    V2 = (q2[0].reshape(E0, H0, I0 // 2), q2[1].reshape(E0, H0, I0 // 16), q2[2])
    rec = {"tokens": w0.tokens}
    for th in (cores, 1):
        d0, st0 = _oracle_layer(O, w0, V1, V2, w0.tokens, th)
        rec[f"threads_{th}"] = {"value": w0.tokens / d0, "unit": "tokens/s", "wall_s": round(d0, 4),
                                "stage_s": st0}
    extra[w0.name] = rec
    w3 = make_moe(3, with_weights=False)
    rec = {"weights": "the headline workload's (same shapes and distribution)"}
    for th, nt in ((cores, w3.tokens), (1, 32)):
        d3, st3 = _oracle_layer(O, w3, W1, W2, nt, th)
        rec[f"threads_{th}"] = {"tokens": nt, "value": nt / d3, "unit": "tokens/s",
                                "wall_s": round(d3, 3), "stage_s": st3}
    extra[w3.name] = rec
    O.set_num_threads(cores)
    log(f"cpu baseline: extra lines {json.dumps(extra)}")
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n_tokens} of {w.tokens} tokens of the same workload (same routing "
                      f"and weights), whole layer: route+quantize, FC1, SwiGLU, requantize, FC2, "
                      f"combine; one run, {dt:.2f} s wall on {cores} threads",
            "runs": 1, "stage_s": stages, "extra": extra}


def main():
    args = parse()
    SETTLE["max_steps"] = max(0, args.settle_max_steps)
    if args.gpus != 1:
        print(f"bench.py: the expert layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is designed, not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch

    from nvfp4_w4a4_quantized_amd.ops import (NvFp4Weights, StageTimer, moe_expert_forward,
                                              moe_expert_forward_workspace_size)
    from nvfp4_w4a4_quantized_amd.workloads import make_moe

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    log(f"generating workload {args.workload}")
    w = make_moe(args.workload)
    fc1_flops, fc2_flops, qbytes = moe_algorithmic(w)

    def bf(u16):
        return torch.from_numpy(u16.view(np.int16)).to(dev).view(torch.bfloat16)

    x = bf(w.x)
    idx = torch.from_numpy(w.topk_idx).to(dev)
    prob = torch.from_numpy(w.topk_prob).to(dev)
    log("quantizing weights and moving them to the GEMM's tiled layout (a0, offline)")
    W1 = NvFp4Weights.quantize(bf(w.w1)).packed()
    W2 = NvFp4Weights.quantize(bf(w.w2)).packed()
    ws = torch.empty(moe_expert_forward_workspace_size(w.tokens, w.hidden, w.inter, w.topk,
                                                       w.experts), dtype=torch.uint8, device=dev)
    y = torch.empty((w.tokens, w.hidden), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def timed(W1, W2, rule):
        def step(timer):
            moe_expert_forward(x, idx, prob, w.experts, w.inter, W1, W2, workspace=ws, y=y,
                               timer=timer, act_block_rule=rule)
        # throughput from the steps exactly as a caller runs them (no events
        # between the stages: each recorded event idles the GPU ~5 us); the
        # per-stage breakdown and the FC1 roofline from the same number of
        # steps again with HIP events recorded on the launch stream
        return run_steps(step, args.steps, args.warmup, f"block rule {rule}", StageTimer)

    if args.skip_headline:
        secondary = run_secondary(args, dev, bf, W1, W2)
        print(json.dumps({"metric": "MoE W4A4 expert-layer tokens/s", "value": None,
                          "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
                          "warmup": args.warmup, "note": "headline skipped (profiling aid)",
                          "secondary": secondary}), flush=True)
        return
    wall, stages = timed(W1, W2, 0)
    ms = wall * 1e3 / args.steps
    tokens_per_s = w.tokens * args.steps / wall
    total_flops = fc1_flops + fc2_flops
    fc1_ms = stages["fc1_swiglu"]
    fc1_tflops = fc1_flops / (fc1_ms * 1e-3) / 1e12
    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        from nvfp4_w4a4_quantized_amd.traffic import gemm_source_hash
        with open(args.traffic) as f:
            rec = json.load(f)
        if rec.get("gemm_source_sha256") == gemm_source_hash() and rec.get("workload") == w.name:
            traffic = rec.get("fc1_hbm_bytes_per_launch")
    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.int32, device=dev).fill_(1)
        dst = torch.empty(n, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        for _ in range(3):   # a plain elementwise kernel: reads n*4 bytes, writes n*4 bytes
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 elementwise copies of {args.copy_calib_mib} MiB")
    log("stages (ms, HIP events): " + ", ".join(f"{k}={v:.4f}" for k, v in stages.items()))
    result = {
        "metric": "MoE W4A4 expert-layer tokens/s",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 e2m1/e4m3 operands decoded exactly to f16 for f16 MFMA, f32 accumulate",
        "data": "synthetic (seeded; Qwen3-30B-A3B expert-layer shapes, random N(0,0.02) weights)",
        "config": {"workload": w.name, "tokens": w.tokens, "hidden": w.hidden,
                   "moe_intermediate": w.inter, "experts": w.experts, "topk": w.topk,
                   "router": f"softmax(N(0,1) + Zipf(s={w.meta['zipf_s']}) bias), top-k renormalised",
                   "routed_rows": w.routed_rows, "active_experts": w.meta["active_experts"],
                   "cv_rows_per_expert": round(w.meta["cv_rows_per_expert"], 3),
                   "parallelism": "single GPU"},
        "effective_tflops": total_flops / (ms * 1e-3) / 1e12,
        "effective_frac_of_f16_peak": total_flops / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS,
        "stage_ms": stages,
        "stage_sum_ms": float(sum(stages.values())),
        "route_quantize_bytes": layer_route_bytes(w),
        "route_quantize_gbps": layer_route_bytes(w) / (stages["route_quantize"] * 1e-3) / 1e9,
        "moe_permute": bench_permute(args, w, x, idx, prob, qbytes),
        "roofline": {"kernel": "FC1 grouped GEMM + SwiGLU/amax epilogue",
                     "bound": "mfma", "achieved": fc1_tflops, "peak": PEAK_F16_TFLOPS,
                     "unit": "TFLOP/s", "frac": fc1_tflops / PEAK_F16_TFLOPS,
                     "traffic": traffic,
                     "per_launch_flops": fc1_flops},
    }
    if args.four_over_six:
        log("Four-Over-Six (MSE): weights requantized offline, activations in the layer")
        V1 = NvFp4Weights.quantize(bf(w.w1), block_rule=1).packed()
        V2 = NvFp4Weights.quantize(bf(w.w2), block_rule=1).packed()
        wall46, st46 = timed(V1, V2, 1)
        log("stages 4/6 (ms, HIP events): " + ", ".join(f"{k}={v:.4f}" for k, v in st46.items()))
        result["four_over_six"] = {
            "block_rule": "4/6, block error = sum of squares",
            "value": w.tokens * args.steps / wall46, "unit": "tokens/s",
            "ms_per_step": wall46 * 1e3 / args.steps, "stage_ms": st46,
            "route_quantize_gbps": layer_route_bytes(w) / (st46["route_quantize"] * 1e-3) / 1e9,
        }
    if args.single_pass:
        result["single_pass"] = bench_single_pass(args, w, x, idx, prob, W1, W2)
    if args.backward:
        result["backward"] = bench_backward(args, w, x, idx, prob, W1, W2, bf)
    sec = run_secondary(args, dev, bf, W1, W2)
    if sec:
        result["secondary"] = sec
    # offline weight quantization (a0) of W1: 1D blocks and 16x16 blocks.  Five
    # calls back to back after a warm-up call, so that the launches queue
    # ahead of the GPU and the figure is the GPU time per call (group amax,
    # scale finalisation, encode), not the host's allocation gaps.
    wq = {}
    wb = bf(w.w1)
    for name, kw in (("w1_1d", {}), ("w1_2d", {"blocks_2d": True})):
        NvFp4Weights.quantize(wb, **kw)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            NvFp4Weights.quantize(wb, **kw)
        e1.record()
        torch.cuda.synchronize()
        wq[name] = e0.elapsed_time(e1) / 5
    result["weight_quantize_ms"] = wq
    if args.cpu_tokens > 0:
        result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_tokens, w.tokens))
    else:
        result["cpu_baseline"] = None
    result["clock_settle"] = {
        "note": ("after the requested warm-up, extra untimed steps in batches of "
                 f"{SETTLE_BATCH} until a batch's step time is within {SETTLE_TOL:.0%} of the "
                 f"previous batch (at most {SETTLE['max_steps']}): the GPU clock ramps over the "
                 "first few hundred milliseconds of sustained work"),
        **SETTLE_LOG}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
