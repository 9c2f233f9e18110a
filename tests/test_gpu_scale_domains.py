"""GPU parity of the extra outer-scale domains through the C ABI: 16x16
two-dimensional weight blocks (scale domain 2) and the per-tensor scale (one
group over all rows), bit for bit against the oracle; a layer run on 2D
weights against the oracle layer on the same weights; the layer with one
activation outer scale per tensor as a replay chain."""
import numpy as np
import pytest
import torch

from gpu_util import assert_gemm_close, dev, dev_bf16, host, moe_case, say
from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, random_bf16
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _ops():
    from nvfp4_w4a4_quantized_amd import ops
    return ops


def _same(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    assert np.array_equal(a, b), what


@pytest.mark.parametrize("shape", [(1, 16, 16), (3, 48, 96), (2, 256, 2048), (4, 2048, 768)])
def test_2d_blocks_match_oracle(shape):
    G, N, K = shape
    rng = np.random.default_rng(N + K)
    w = random_bf16(rng, (G, N, K), 0.02)
    w[0, :16, :16] = 0                                   # an all-zero tile
    offs = np.arange(G + 1, dtype=np.int32) * N
    say("2D blocks", shape)
    c, s, g = _ops().nvfp4_quantize(dev_bf16(w.reshape(G * N, K)), scale_domain=2,
                                    group_offsets=dev(offs))
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(w.reshape(G * N, K), domain=2, group_offsets=offs)
    _same(host(g), rg, "outer scales")
    _same(host(s), rs, "scales")
    _same(host(c), rc, "codes")


def test_per_tensor_scale_matches_oracle():
    rng = np.random.default_rng(71)
    x = random_bf16(rng, (300, 512), 1.0)
    offs = np.array([0, 300], np.int32)
    say("per-tensor scale")
    c, s, g = _ops().nvfp4_quantize(dev_bf16(x), scale_domain=1, group_offsets=dev(offs))
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(x, domain=1, group_offsets=offs)
    _same(host(g), rg, "outer scale")
    _same(host(s), rs, "scales")
    _same(host(c), rc, "codes")


def test_layer_on_2d_weights():
    """The grouped GEMMs read 2D-block weights unchanged: FC1 within the GEMM
    tolerance of the oracle on the same operands, y close to the oracle layer."""
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights, moe_expert_forward, w4a4_grouped_gemm
    w, _, _ = moe_case(0)
    E, I = w.experts, w.inter
    W1 = NvFp4Weights.quantize(dev_bf16(w.w1), blocks_2d=True)
    W2 = NvFp4Weights.quantize(dev_bf16(w.w2), blocks_2d=True)
    OW1 = tuple(host(t) for t in (W1.codes, W1.scales, W1.gscale))
    OW2 = tuple(host(t) for t in (W2.codes, W2.scales, W2.gscale))
    ref1 = O.quantize(w.w1.reshape(-1, w.w1.shape[2]), domain=2,
                      group_offsets=np.arange(E + 1, dtype=np.int32) * 2 * I)
    _same(OW1[1].reshape(-1, OW1[1].shape[2]), ref1[1], "W1 2D scales")
    p = O.moe_permute(w.x, w.topk_idx, w.topk_prob, E)
    offs = p["offsets"]
    say("gemm on 2D weights")
    out = w4a4_grouped_gemm(dev(p["codes"]), dev(p["scales"]), dev(p["gscale"]), W1.packed(),
                            dev(offs))
    torch.cuda.synchronize()
    R = int(offs[-1])
    cref, cb = O.grouped_gemm(p["codes"], p["scales"], p["gscale"], *OW1, offs, with_bound=True)
    assert_gemm_close(host(out)[:R], cref[:R], cb[:R], "FC1 on 2D weights")
    say("layer on 2D weights")
    y = moe_expert_forward(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), E, I, W1, W2)
    torch.cuda.synchronize()
    yo, _ = O.moe_forward(w.x, w.topk_idx, w.topk_prob, E, I, OW1, OW2)
    a = bf16_bits_to_f32(host(y)).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel < 1e-2, rel


@pytest.mark.parametrize("wid,align,rule", [(0, 16, 0), (3, 1, 0), (0, 1, 1)])
def test_layer_per_tensor_activation_scale(wid, align, rule):
    """moe_expert_forward with one activation outer scale per tensor
    (act_scale_domain 1), as a replay chain against the oracle: the routed A1
    rows are the oracle's per-tensor quantization of x (domain 1, one group
    over all tokens) bit for bit, FC1 and FC2 every element within the GEMM
    tolerance, A2 the oracle's per-tensor quantization of the GPU's D with the
    maximum of its row amax bit for bit, y the combine of the FC2 rows."""
    from gpu_util import assert_gemm_full, bf16_ulp
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights, moe_expert_forward
    w, W1, W2 = moe_case(wid)
    T = w.tokens
    say("per-tensor activation scale layer", w.name, "align", align, "rule", rule)
    wq = [NvFp4Weights(dev(W[0]), dev(W[1]), dev(W[2])) for W in (W1, W2)]
    y, it = moe_expert_forward(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts,
                               w.inter, wq[0], wq[1], align=align, debug=True, fc1_out=True,
                               y_rows_f32=True, act_block_rule=rule, act_scale_domain=1)
    torch.cuda.synchronize()
    y = host(y)
    it = {k: host(v) for k, v in it.items()}
    off = it["expert_offsets"]
    R = int(off[-1])
    rs = it["row_src"][:R]
    routed = rs >= 0
    # A1: the tokens' per-tensor quantization, permuted
    tc, ts, tg = O.quantize(w.x, domain=1, group_offsets=np.array([0, T], np.int32), rule=rule)
    _same(it["a1_codes"][:R][routed], tc[rs[routed]], "A1 codes")
    _same(it["a1_scales"][:R][routed], ts[rs[routed]], "A1 scales")
    assert not it["a1_codes"][:R][~routed].any() and not it["a1_scales"][:R][~routed].any()
    _same(it["a1_gscale"][:R][routed], np.full(routed.sum(), tg[0], np.float32), "A1 outer scale")
    A1 = (it["a1_codes"], it["a1_scales"], it["a1_gscale"])
    C = it["fc1_out"][:R]
    assert_gemm_full(C, A1, W1, off, "FC1 (per-tensor A1)")
    D = it["d"][:R]
    dref, _ = O.swiglu(C, it["row_prob"][:R])
    dv = bf16_bits_to_f32(D).astype(np.float64)
    rv = bf16_bits_to_f32(dref).astype(np.float64)
    assert np.all(np.abs(dv - rv) <= bf16_ulp(rv) * 1.0001 + 1e-40), "SwiGLU D"
    amax = it["amax_d"][:R]
    assert np.array_equal(amax, np.abs(bf16_bits_to_f32(D)).max(axis=1)), "amax_d"
    # A2: one scale from the largest row amax
    tamax = np.array([amax.max() if R else 0.0], np.float32)
    c2, s2, g2 = O.quantize(D, domain=1, group_offsets=np.array([0, R], np.int32),
                            amax_in=tamax, rule=rule)
    _same(it["a2_codes"][:R], c2, "A2 codes")
    _same(it["a2_scales"][:R], s2, "A2 scales")
    _same(it["a2_gscale"][:R], np.full(R, g2[0], np.float32), "A2 outer scale")
    A2 = (it["a2_codes"], it["a2_scales"], it["a2_gscale"])
    Y = it["y_rows_f32"][:R]
    assert_gemm_full(Y, A2, W2, off, "FC2 (per-tensor A2)")
    ycomb = bf16_bits_to_f32(O.combine(Y, it["dst_row"])).astype(np.float64)
    yv = bf16_bits_to_f32(y).astype(np.float64)
    absum = np.zeros_like(yv)
    dst = it["dst_row"]
    for j in range(dst.shape[1]):
        ok = dst[:, j] >= 0
        absum[ok] += np.abs(Y[dst[ok, j]])
    tol = absum * 2.0 ** -20 + bf16_ulp(ycomb) * 1.0001 + 1e-30
    assert np.all(np.abs(yv - ycomb) <= tol), "combine"
