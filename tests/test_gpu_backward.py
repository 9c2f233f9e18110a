"""moe_expert_backward through the C ABI, checked against oracle/backward.py.

The forward runs first (moe_expert_forward with its intermediates) to give
the routing, the FC1 output C and the FC2 input D.  Every backward step is
then compared on the inputs the GPU itself produced upstream (a replay
chain), so one bf16 rounding flip is not compounded:
  dD   (bf16)  vs the oracle dgrad of dYr and W2: fp32 GEMM bound plus one
               bf16 ulp
  dC   (bf16)  vs the oracle SwiGLU backward of the GPU's dD: one bf16 ulp
               plus the fp32 evaluation of sigmoid
  dp   (fp32)  vs the oracle's row sums on the GPU's dD: fp32 sum bound
  dXr  (fp32)  vs the oracle dgrad of the GPU's dC and W1: fp32 GEMM bound;
               the bf16 rows are the round-to-nearest-even of the fp32 ones
  dx           bit-exact: the fp32 sum of the bf16 rows in entry order
  dprob        bit-exact: the entry's row sum
  dW2, dW1     vs the oracle wgrads: fp32 GEMM bound per expert
and end to end against the oracle's whole backward in float64 (relative L2:
dx, dW1 and dprob carry the bf16 roundings of dD, dC and dXr).

fp32 GEMM bound: bf16 x bf16 products are exact in fp32; K of them summed in
fp32 in any order stay within (K + 16) 2^-24 sum |a b| of the exact sum (the
sequential-summation bound with margin).
"""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, oracle_weights, say
from nvfp4_w4a4_quantized_amd.workloads import (MoeWorkload, bf16_bits_to_f32, make_moe,
                                                random_bf16, route_topk, to_bf16_bits)
from oracle import backward as B
from oracle import oracle as O

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _custom(seed, T, H, I, E, k, zipf=0.0, banned=()):
    """A synthetic MoE workload of the given shape (router logits N(0,1) plus
    a Zipf-like bias; `banned` experts receive no tokens)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    logits = rng.standard_normal((T, E), dtype=np.float32)
    if zipf:
        logits += (-zipf * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)
    for e in banned:
        logits[:, e] = -np.inf
    idx, prob = route_topk(logits, k)
    x = random_bf16(rng, (T, H))
    w1 = random_bf16(rng, (E, 2 * I, H), 0.02)
    w2 = random_bf16(rng, (E, H, I), 0.02)
    return MoeWorkload(f"bwd_T{T}_H{H}_I{I}_E{E}_k{k}", -1, T, H, I, E, k, x, idx, prob, w1, w2)


def _forward(w, W1q, W2q, align):
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights, moe_expert_forward
    say("moe_expert_forward (for the backward)", w.name, "align", align)
    wq = [NvFp4Weights(dev(W[0]), dev(W[1]), dev(W[2])) for W in (W1q, W2q)]
    _, it = moe_expert_forward(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts,
                               w.inter, wq[0], wq[1], align=align, debug=True, fc1_out=True)
    return it


def _dequantized_bf16(Wq, shape):
    G, N, K = shape
    v = O.dequantize(Wq[0].reshape(G * N, K // 2), Wq[1].reshape(G * N, K // 16),
                     np.repeat(Wq[2], N))
    return to_bf16_bits(v.astype(np.float32)).reshape(shape)


def _backward(w, it, dy, w1b, w2b, **kw):
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_backward
    say("moe_expert_backward", w.name, kw)
    out, dbg = moe_expert_backward(dev_bf16(dy), dev_bf16(w.x), it["fc1_out"], it["d"],
                                   it["expert_offsets"], it["row_src"], it["row_prob"],
                                   it["dst_row"], dev_bf16(w1b), dev_bf16(w2b), debug=True,
                                   dx_rows_f32=True, **kw)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in out.items()}, {k: host(v) for k, v in dbg.items()}


def _close(gpu, ref, tol, what):
    err = np.abs(np.asarray(gpu, np.float64) - ref)
    bad = np.flatnonzero(~(err <= tol))
    assert bad.size == 0, (f"{what}: {bad.size} of {err.size} outside tolerance; first idx "
                           f"{bad[:4]}, gpu {np.asarray(gpu).reshape(-1)[bad[:4]]}, ref "
                           f"{ref.reshape(-1)[bad[:4]]}, tol {np.broadcast_to(tol, ref.shape).reshape(-1)[bad[:4]]}")


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _check_chain(w, it_dev, out, dbg, w1b, w2b, dy):
    """The replay chain; returns the host copies of the forward's arrays."""
    it = {k: host(v) for k, v in it_dev.items()}
    off = it["expert_offsets"].astype(np.int64)
    R = int(off[-1])
    H, I = w.hidden, w.inter
    row_src = it["row_src"][:R]
    pad = row_src < 0
    W1 = B.bf16(w1b)
    W2 = B.bf16(w2b)
    dYr = B.gather_rows(B.bf16(dy), row_src, R)
    # dD: the fp32 GEMM bound, then one bf16 rounding
    ref, babs = B.grouped_dgrad(dYr, W2, off)
    dd = B.bf16(dbg["dd"][:R])
    _close(dd, ref, (H + 16) * U32 * babs + 2.0 ** -7 * np.abs(ref) + 1e-38, "dD")
    # dC and dp on the GPU's dD
    C = it["fc1_out"][:R].astype(np.float64)
    p = it["row_prob"][:R].astype(np.float64)
    p[pad] = 0.0
    ref_dc, ref_dp = B.swiglu_backward(dd, C, p)
    ref_dc[pad] = 0.0
    ref_dp[pad] = 0.0
    g, u = C[:, :I], C[:, I:]
    pp = np.abs(p)[:, None]
    ag = np.abs(g)
    sig = 1.0 / (1.0 + np.exp(-g))
    tol_g = 2.0 ** -7 * np.abs(ref_dc[:, :I]) + 2.0 ** -18 * np.abs(dd * u) * pp * (1 + ag) ** 2
    tol_u = 2.0 ** -7 * np.abs(ref_dc[:, I:]) + 2.0 ** -18 * np.abs(dd * g) * pp * (1 + ag)
    dc = B.bf16(dbg["dc"][:R])
    _close(dc[:, :I], ref_dc[:, :I], tol_g + 1e-38, "dC gate")
    _close(dc[:, I:], ref_dc[:, I:], tol_u + 1e-38, "dC up")
    s1 = np.sum(np.abs(dd * g * sig * u), axis=1)
    s2 = np.sum(np.abs(dd * u * g) * (1 + ag), axis=1)
    _close(dbg["dp_rows"][:R], ref_dp, (I + 16) * U32 * s1 + 2.0 ** -18 * s2 + 1e-38, "dp rows")
    # dXr on the GPU's dC
    ref, babs = B.grouped_dgrad(dc, W1, off)
    _close(dbg["dx_rows_f32"][:R], ref, (2 * I + 16) * U32 * babs + 1e-30, "dXr")
    assert np.array_equal(dbg["dx_rows"][:R], to_bf16_bits(dbg["dx_rows_f32"][:R])), "dXr bf16"
    # dx: fp32 sums of the bf16 rows in entry order, then bf16
    dst = it["dst_row"]
    rows32 = bf16_bits_to_f32(dbg["dx_rows"])
    acc = np.zeros((w.tokens, H), np.float32)
    for j in range(w.topk):
        ok = dst[:, j] >= 0
        acc[ok] += rows32[dst[ok, j]]
    assert np.array_equal(out["dx"], to_bf16_bits(acc)), "dx"
    # dprob: the entry's row sum, bit for bit
    exp = np.where(dst >= 0, dbg["dp_rows"][np.maximum(dst, 0)], np.float32(0.0))
    assert np.array_equal(out["dprob"].view(np.uint32), exp.astype(np.float32).view(np.uint32))
    # wgrads, per expert
    D = B.bf16(it["d"][:R])
    ref2, babs2 = B.grouped_wgrad(dYr, D, off)
    Xr = B.gather_rows(B.bf16(w.x), row_src, R)
    ref1, babs1 = B.grouped_wgrad(dc, Xr, off)
    for e in range(w.experts):
        K = int(off[e + 1] - off[e])
        _close(out["dw2"][e], ref2[e], (K + 16) * U32 * babs2[e] + 1e-30, f"dW2[{e}]")
        _close(out["dw1"][e], ref1[e], (K + 16) * U32 * babs1[e] + 1e-30, f"dW1[{e}]")
        if K == 0:
            assert not out["dw1"][e].any() and not out["dw2"][e].any(), f"empty expert {e}"
    return it


def _end_to_end(w, it, out, w1b, w2b, dy):
    off = it["expert_offsets"]
    R = int(off[-1])
    row_src = it["row_src"][:R]
    p = it["row_prob"][:R].astype(np.float64)
    p[row_src < 0] = 0.0
    ref, _ = B.moe_backward(B.bf16(dy), B.bf16(w.x), it["fc1_out"][:R].astype(np.float64),
                            B.bf16(it["d"][:R]), row_src, p, off, it["dst_row"],
                            B.bf16(w1b), B.bf16(w2b))
    errs = {
        "dx": _rel_l2(B.bf16(out["dx"]), ref["dx"]),
        "dw1": _rel_l2(out["dw1"], ref["dW1"]),
        "dw2": _rel_l2(out["dw2"], ref["dW2"]),
        "dprob": _rel_l2(out["dprob"], ref["dprob"]),
    }
    say("backward relative L2 vs the float64 oracle", errs)
    # dx, dW1 and dprob carry bf16 roundings of dD, dC (and dXr), each within
    # 2^-8 relative; dW2 only fp32 accumulation
    assert errs["dx"] < 1e-2 and errs["dw1"] < 1e-2 and errs["dprob"] < 1e-2, errs
    assert errs["dw2"] < 1e-4, errs


CASES = {
    # several m-tiles per expert, a ragged 128-column FC2 n-tile, padding rows
    "t1024_h512_i384_e16_k4_align16": dict(seed=71, T=1024, H=512, I=384, E=16, k=4, align=16),
    # skewed routing, one row alignment, two experts left empty
    "t512_h256_i256_e8_k2_empty": dict(seed=72, T=512, H=256, I=256, E=8, k=2, align=1,
                                       zipf=1.2, banned=(3, 7)),
    # hidden 384: FC2's wgrad has a 256-row output tile half past its rows and
    # FC1's dgrad a 256-column tile half past its columns
    "t384_h384_i128_e4_k2": dict(seed=73, T=384, H=384, I=128, E=4, k=2, align=1),
    # the largest hidden and intermediate sizes
    "t96_h16384_i128_e4_k2": dict(seed=74, T=96, H=16384, I=128, E=4, k=2, align=1),
    "t96_h256_i16384_e4_k2": dict(seed=75, T=96, H=256, I=16384, E=4, k=2, align=1),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("operands", ["saved_bf16", "dequantized"])
def test_backward_replay_chain(name, operands):
    c = dict(CASES[name])
    align = c.pop("align")
    w = _custom(**c)
    W1q, W2q = oracle_weights(w.w1), oracle_weights(w.w2)
    if operands == "saved_bf16":
        w1b, w2b = w.w1, w.w2
    else:
        w1b = _dequantized_bf16(W1q, w.w1.shape)
        w2b = _dequantized_bf16(W2q, w.w2.shape)
    it_dev = _forward(w, W1q, W2q, align)
    dy = random_bf16(np.random.Generator(np.random.PCG64(c["seed"] + 1000)), (w.tokens, w.hidden))
    out, dbg = _backward(w, it_dev, dy, w1b, w2b)
    it = _check_chain(w, it_dev, out, dbg, w1b, w2b, dy)
    _end_to_end(w, it, out, w1b, w2b, dy)


def test_backward_tiny_workload_and_determinism():
    w = make_moe(0)
    W1q, W2q = oracle_weights(w.w1), oracle_weights(w.w2)
    it_dev = _forward(w, W1q, W2q, 16)
    dy = random_bf16(np.random.Generator(np.random.PCG64(5)), (w.tokens, w.hidden))
    out, dbg = _backward(w, it_dev, dy, w.w1, w.w2)
    it = _check_chain(w, it_dev, out, dbg, w.w1, w.w2, dy)
    _end_to_end(w, it, out, w.w1, w.w2, dy)
    out2, _ = _backward(w, it_dev, dy, w.w1, w.w2)
    for k in out:
        assert np.array_equal(out[k].view(np.uint8), out2[k].view(np.uint8)), k


def test_backward_no_tokens():
    """No routed rows: every expert's weight gradient is zero."""
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_backward
    E, H, I = 4, 256, 128
    say("moe_expert_backward with no tokens")
    z = lambda shape, dt: torch.zeros(shape, dtype=dt, device="cuda")  # noqa: E731
    w1 = dev_bf16(random_bf16(np.random.Generator(np.random.PCG64(3)), (E, 2 * I, H), 0.02))
    w2 = dev_bf16(random_bf16(np.random.Generator(np.random.PCG64(4)), (E, H, I), 0.02))
    out = dict(dx=z((0, H), torch.bfloat16), dw1=torch.full((E, 2 * I, H), 7.0, device="cuda"),
               dw2=torch.full((E, H, I), 7.0, device="cuda"), dprob=z((0, 2), torch.float32))
    moe_expert_backward(z((0, H), torch.bfloat16), z((0, H), torch.bfloat16),
                        z((0, 2 * I), torch.float32), z((0, I), torch.bfloat16),
                        z(E + 1, torch.int32), z(0, torch.int32), z(0, torch.float32),
                        z((0, 2), torch.int32), w1, w2, out=out)
    torch.cuda.synchronize()
    assert not out["dw1"].any().item() and not out["dw2"].any().item()


def test_backward_qwen3_moe_t8192_full():
    """The Qwen3-30B-A3B-shaped layer at 8192 tokens: the whole replay chain
    (every element of every output) and the end-to-end check."""
    w = make_moe(2)
    W1q, W2q = oracle_weights(w.w1), oracle_weights(w.w2)
    it_dev = _forward(w, W1q, W2q, 1)
    dy = random_bf16(np.random.Generator(np.random.PCG64(2002)), (w.tokens, w.hidden))
    out, dbg = _backward(w, it_dev, dy, w.w1, w.w2)
    say("checking the t8192 backward on the host")
    it = _check_chain(w, it_dev, out, dbg, w.w1, w.w2, dy)
    _end_to_end(w, it, out, w.w1, w.w2, dy)
