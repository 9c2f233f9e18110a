"""moe_expert_forward_single_pass (FC1 -> weighted SwiGLU -> online-amax
NVFP4 quantization -> FC2 in one kernel; miniTE Technical Report §5.6)
through the C ABI, as a replay chain against the oracle's O12:
  routing, A1           bit-exact (as the two-pass layer)
  FC1 C (fp32)          every element within the GEMM tolerance
  P (bf16 SwiGLU)       within one bf16 ulp of the oracle SwiGLU of the GPU's C
  online quantization   codes, E4M3 scales and per-tile gs bit-exact against
                        O12a applied to the GPU's own P
  FC2 rows              every element within 2^-10 * sum|a_k b_k| + 1e-6 of
                        O12b on the GPU's own online quantization
  combine               within the summed bounds
and, loosely, y against a pure oracle run of the single-pass layer.  A layer
whose intermediate size is one tile is the two-pass layer, bit for bit."""
import numpy as np
import pytest
import torch

from gpu_util import (assert_gemm_full, bf16_ulp, dev, dev_bf16, fc1_oracle_chunks, host,
                      moe_case, oracle_single_pass_chunks, oracle_weights, say)
from nvfp4_w4a4_quantized_amd.workloads import MoeWorkload, bf16_bits_to_f32, random_bf16, route_topk
from oracle import oracle as O

pytestmark = pytest.mark.gpu

TILE = 256


def _weights(W, tiled=False):
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights
    w = NvFp4Weights(dev(W[0]), dev(W[1]), dev(W[2]))
    return w.packed() if tiled else w


def _run(w, W1, W2, align=1, tiled=False, **kw):
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_forward_single_pass
    say("single-pass layer", w.name, "align", align, "tiled" if tiled else "row-major", kw)
    y, it = moe_expert_forward_single_pass(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob),
                                           w.experts, w.inter, _weights(W1, tiled),
                                           _weights(W2, tiled), align=align, debug=True, **kw)
    torch.cuda.synchronize()
    return host(y), {k: host(v) for k, v in it.items()}


def _replay(w, W1, W2, align=1, tiled=False, fc1_chunks=None):
    y, it = _run(w, W1, W2, align, tiled, fc1_out=True, y_rows_f32=True)
    ref = O.moe_permute(w.x, w.topk_idx, w.topk_prob, w.experts, align)
    off = it["expert_offsets"]
    assert np.array_equal(off, ref["offsets"])
    assert np.array_equal(it["dst_row"], ref["dst_row"])
    R = int(off[-1])
    for a, b in (("a1_codes", "codes"), ("a1_scales", "scales"), ("a1_gscale", "gscale")):
        assert np.array_equal(it[a][:R].view(np.uint8), ref[b][:R].view(np.uint8)), a
    A1 = (it["a1_codes"], it["a1_scales"], it["a1_gscale"])
    C = it["fc1_out"][:R]
    assert_gemm_full(C, A1, W1, off, "single-pass FC1", chunks=fc1_chunks)
    P = it["p"][:R]
    pref, _ = O.swiglu(C, it["row_prob"][:R])
    pv = bf16_bits_to_f32(P).astype(np.float64)
    rv = bf16_bits_to_f32(pref).astype(np.float64)
    assert np.all(np.abs(pv - rv) <= bf16_ulp(rv) * 1.0001 + 1e-40), "SwiGLU P"
    codes, scales, gs = O.online_quantize(P, TILE)
    assert np.array_equal(it["a2_codes"][:R], codes), "online codes"
    assert np.array_equal(it["a2_scales"][:R], scales), "online scales"
    assert np.array_equal(it["gs_tiles"][:R].view(np.uint32), gs.view(np.uint32)), "tile gs"
    Y = it["y_rows_f32"][:R]
    A2 = (it["a2_codes"], it["a2_scales"])
    chunks = list(oracle_single_pass_chunks(A2, it["gs_tiles"], TILE, W2, off))
    assert_gemm_full(Y, None, W2, off, "single-pass FC2", chunks=chunks)
    ycomb = bf16_bits_to_f32(O.combine(Y, it["dst_row"])).astype(np.float64)
    yv = bf16_bits_to_f32(y).astype(np.float64)
    absum = np.zeros_like(yv)
    dst = it["dst_row"]
    for j in range(dst.shape[1]):
        ok = dst[:, j] >= 0
        absum[ok] += np.abs(Y[dst[ok, j]])
    assert np.all(np.abs(yv - ycomb) <= absum * 2.0 ** -20 + bf16_ulp(ycomb) * 1.0001 + 1e-30)
    return y, it


def _end_to_end(w, W1, W2, y, align=1):
    yo, _ = O.moe_forward_single_pass(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2,
                                      tile=TILE, align=align)
    a = bf16_bits_to_f32(y).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    rel = np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30)
    print(f"{w.name}: single-pass layer end-to-end rel L2 vs pure oracle run {rel:.3e}")
    assert rel < 1e-2


def test_one_tile_layer_is_the_two_pass_layer():
    """Intermediate 128 (one tile): the online scale is the row amax, so the
    codes, scales and FC2 arithmetic are the two-pass layer's; y matches bit
    for bit."""
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_forward
    w, W1, W2 = moe_case(0)
    y, it = _replay(w, W1, W2)
    y2 = moe_expert_forward(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts, w.inter,
                            _weights(W1), _weights(W2))
    torch.cuda.synchronize()
    yd, _ = _run(w, W1, W2)                       # bf16 FC2 rows, as the two-pass layer
    assert np.array_equal(yd, host(y2))
    _end_to_end(w, W1, W2, y)


def _multi_tile_case(tokens, experts, H, I, k, seed, zipf=1.1):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((tokens, experts)).astype(np.float32)
    logits += (-zipf * np.log(np.arange(1, experts + 1))).astype(np.float32)
    idx, prob = route_topk(logits, k)
    x = random_bf16(rng, (tokens, H))
    x[5] = 0                                      # an all-zero row: gs = 0 in every tile
    w = MoeWorkload(f"single_pass_t{tokens}_i{I}", -1, tokens, H, I, experts, k, x, idx, prob,
                    None, None, {})
    W1 = oracle_weights(random_bf16(rng, (experts, 2 * I, H), 0.02))
    W2 = oracle_weights(random_bf16(rng, (experts, H, I), 0.02))
    return w, W1, W2


@pytest.mark.parametrize("I,align,tiled", [(768, 1, True), (384, 16, False), (640, 1, False),
                                            (1152, 1, True)])
def test_multi_tile_replay_chain(I, align, tiled):
    """Three tiles (768), a full and a half tile (384: 256 + 128), three
    tiles ending in a half one (640), the largest intermediate size with
    its FC2 input filling the LDS (1152: four tiles and a half); padding
    rows; both weight layouts."""
    w, W1, W2 = _multi_tile_case(700, 16, 256, I, 4, I + align)
    y, it = _replay(w, W1, W2, align, tiled)
    R = int(it["expert_offsets"][-1])
    gs = it["gs_tiles"][:R]
    # the running amax: non-decreasing, and it grows in some rows
    assert np.all(np.diff(gs, axis=1) >= 0)
    assert np.any(gs[:, -1] > gs[:, 0])
    _end_to_end(w, W1, W2, y, align)


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_workload_replay_chain(wid):
    """The Qwen3-shaped (three tiles per row), decode-shaped and long
    heavy-tail layers (zero rows: all tiles skipped; Student-t activations)
    at full size, every FC1 and FC2 element."""
    w, W1, W2 = moe_case(wid)
    y, it = _replay(w, W1, W2, tiled=(wid == 2), fc1_chunks=fc1_oracle_chunks(wid) if wid == 2 else None)
    R = int(it["expert_offsets"][-1])
    gs = it["gs_tiles"][:R]
    changed = float(np.mean(gs[:, -1] != gs[:, 0]))
    print(f"{w.name}: rows whose scale grew after the first tile {changed:.3f}")
    if wid == 3:
        _end_to_end(w, W1, W2, y)


def test_perf_path_and_determinism():
    """The timed configuration (no debug outputs, bf16 FC2 rows, tiled
    weights) gives the same y on repeated calls and as the debug run."""
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_forward_single_pass
    w, W1, W2 = moe_case(2)
    args = (dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts, w.inter,
            _weights(W1, True), _weights(W2, True))
    say("single-pass perf path x2")
    y1 = moe_expert_forward_single_pass(*args)
    y2 = moe_expert_forward_single_pass(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    yd, _ = _run(w, W1, W2, tiled=True)
    assert np.array_equal(yd, host(y1))
