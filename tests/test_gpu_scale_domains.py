"""GPU parity of the extra outer-scale domains through the C ABI: 16x16
two-dimensional weight blocks (scale domain 2) and the per-tensor scale (one
group over all rows), bit for bit against the oracle; a layer run on 2D
weights against the oracle layer on the same weights."""
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
