"""GPU parity of the Four-Over-Six block rule (The 4-bitter Lesson,
"Four-Over-Six for RL Weights and Activations") through the C ABI: codes,
E4M3 scales and outer scales bit for bit against the oracle, for activations,
per-expert weights, the fused quantize-permute and the expert layer."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, moe_case, say
from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, random_bf16, to_bf16_bits
from oracle import oracle as O

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")
RULES = [1, 2]


def _ops():
    from nvfp4_w4a4_quantized_amd import ops
    return ops


def _same(gpu, ref, what):
    gpu = host(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
    ref = np.asarray(ref)
    if gpu.dtype == np.float32:
        gpu, ref = gpu.view(np.uint32), ref.view(np.uint32)
    if not np.array_equal(gpu, ref):
        bad = np.argwhere(gpu != ref)
        raise AssertionError(f"{what}: {len(bad)} entries differ, first at {bad[0].tolist()}")


@pytest.mark.parametrize("rule", RULES)
def test_golden_row(rule):
    with open(os.path.join(GOLD, "four_over_six_row.json")) as f:
        g = json.load(f)
    x = to_bf16_bits(np.array(g["x_values"], np.float32))[None]
    say("4/6 golden row", rule)
    c, s, gs = _ops().nvfp4_quantize(dev_bf16(x), block_rule=rule)
    torch.cuda.synchronize()
    key = "mse" if rule == 1 else "mae"
    assert [f"{b:02x}" for b in host(s)[0]] == g[key]["expected_scales_hex"]
    assert [f"{b:02x}" for b in host(c)[0]] == g[key]["expected_codes_hex"]
    assert f"{host(gs).view(np.uint32)[0]:08x}" == g["expected_gscale_hex"]


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("k", [16, 48, 768, 2048, 4096])
def test_rows_match_oracle(rule, k):
    rng = np.random.default_rng(k + 7 * rule)
    rows = 96
    v = rng.standard_normal((rows, k)).astype(np.float32) * rng.uniform(1e-3, 1e3, (rows, 1))
    v[1] = 0.0
    v[2, ::3] = 5.0                                   # blocks that prefer 4
    v[3] = np.where(rng.random(k) < 0.5, 6.0, 1.0)    # exact lattice values
    v[4] = rng.standard_t(3, k) * 100                  # heavy tails
    x = to_bf16_bits(v.astype(np.float32))
    say("4/6 rows", rule, k)
    c, s, g = _ops().nvfp4_quantize(dev_bf16(x), block_rule=rule)
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(x, rule=rule)
    _same(s, rs, "scales")
    _same(g, rg, "outer scales")
    _same(c, rc, "codes")
    # with the amax supplied (the FC2 requantization path)
    am = np.abs(bf16_bits_to_f32(x)).max(axis=1).astype(np.float32)
    c, s, g = _ops().nvfp4_quantize(dev_bf16(x), amax_in=dev(am), block_rule=rule)
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(x, amax_in=am, rule=rule)
    _same(s, rs, "scales amax_in")
    _same(c, rc, "codes amax_in")


@pytest.mark.parametrize("rule", RULES)
def test_expert_weights(rule):
    w, _, _ = moe_case(0)
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights
    for name, wb in (("w1", w.w1), ("w2", w.w2)):
        G, N, K = wb.shape
        say("4/6 weights", rule, name, wb.shape)
        q = NvFp4Weights.quantize(dev_bf16(wb), block_rule=rule)
        torch.cuda.synchronize()
        rc, rs, rg = O.quantize(wb.reshape(G * N, K), domain=1,
                                group_offsets=np.arange(G + 1, dtype=np.int32) * N, rule=rule)
        _same(q.gscale, rg, f"{name} outer scales")
        _same(q.scales.reshape(G * N, -1), rs, f"{name} scales")
        _same(q.codes.reshape(G * N, -1), rc, f"{name} codes")


@pytest.mark.parametrize("rule", RULES)
def test_permute_matches_oracle(rule):
    w, _, _ = moe_case(2, with_weights=False)
    say("4/6 moe_permute", rule)
    p = _ops().moe_permute(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts,
                           block_rule=rule)
    torch.cuda.synchronize()
    ref = O.moe_permute(w.x, w.topk_idx, w.topk_prob, w.experts, rule=rule)
    R = int(ref["offsets"][-1])
    _same(p["offsets"], ref["offsets"], "offsets")
    _same(host(p["scales"])[:R], ref["scales"][:R], "scales")
    _same(host(p["gscale"])[:R], ref["gscale"][:R], "outer scales")
    _same(host(p["codes"])[:R], ref["codes"][:R], "codes")


def test_expert_layer_replay_with_four_over_six():
    """moe_expert_forward with 4/6 (MSE) activations and 4/6 weights: both
    activation quantizations bit-exact against the oracle (A2 on the GPU's own
    D and amax), y close to a pure oracle run."""
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights, moe_expert_forward
    w, _, _ = moe_case(0)
    rule = 1
    E, I, H = w.experts, w.inter, w.hidden
    W1 = NvFp4Weights.quantize(dev_bf16(w.w1), block_rule=rule)
    W2 = NvFp4Weights.quantize(dev_bf16(w.w2), block_rule=rule)
    say("4/6 moe_expert_forward")
    y, it = moe_expert_forward(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), E, I, W1, W2,
                               debug=True, act_block_rule=rule)
    torch.cuda.synchronize()
    it = {k: host(v) for k, v in it.items()}
    ref = O.moe_permute(w.x, w.topk_idx, w.topk_prob, E, rule=rule)
    R = int(ref["offsets"][-1])
    for a, b in (("a1_codes", "codes"), ("a1_scales", "scales"), ("a1_gscale", "gscale")):
        assert np.array_equal(it[a][:R].view(np.uint8), ref[b][:R].view(np.uint8)), a
    a2 = O.quantize(it["d"][:R], amax_in=it["amax_d"][:R], rule=rule)
    for name, r in zip(("a2_codes", "a2_scales", "a2_gscale"), a2):
        assert np.array_equal(it[name][:R].view(np.uint8), r.view(np.uint8)), name
    OW1 = tuple(host(t) for t in (W1.codes, W1.scales, W1.gscale))
    OW2 = tuple(host(t) for t in (W2.codes, W2.scales, W2.gscale))
    yo, _ = O.moe_forward(w.x, w.topk_idx, w.topk_prob, E, I, OW1, OW2, act_rule=rule)
    a = bf16_bits_to_f32(host(y)).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    print(f"4/6 tiny layer end-to-end rel L2 vs pure oracle: {rel:.3e}")
    assert rel < 1e-2
