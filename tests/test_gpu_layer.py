"""moe_expert_forward end to end (through the C ABI), checked as a replay
chain against the oracle: every step is compared on the inputs the GPU itself
produced upstream, so one rounding flip is not compounded.
  a1/a2  routing + quantized A1: bit-exact vs the oracle
  a3     FC1 C (fp32) vs the oracle GEMM on A1: GEMM tolerance
  a4     D within one bf16 ulp of the oracle SwiGLU of the GPU's C;
         amax_d == max |D| bit-exact
  a5     A2 == oracle quantize(D_gpu, amax_gpu): bit-exact
  a6     FC2 rows vs the oracle GEMM on A2: GEMM tolerance
  a7     y vs the oracle combine of the GPU's FC2 rows: sum of tolerances
and, loosely, y against a pure oracle run (relative L2)."""
import numpy as np
import pytest
import torch

from gpu_util import (assert_gemm_full, bf16_ulp, dev, dev_bf16, fc1_oracle_chunks, host,
                      moe_case, oracle_gemm_chunks, say)
from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _weights(W):
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights
    return NvFp4Weights(dev(W[0]), dev(W[1]), dev(W[2]))


def _forward(w, W1, W2, align=1, tiled=False, **kw):
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_forward
    say("moe_expert_forward", w.name, "align", align, "tiled" if tiled else "row-major", kw)
    w1, w2 = _weights(W1), _weights(W2)
    if tiled:
        w1, w2 = w1.packed(), w2.packed()
    y, it = moe_expert_forward(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts,
                               w.inter, w1, w2, align=align, debug=True, **kw)
    torch.cuda.synchronize()
    return host(y), {k: host(v) for k, v in it.items()}


def _replay_chain(w, W1, W2, align, fc1_chunks=None):
    """Runs the layer with its debug intermediates and checks every step on
    the GPU's own upstream values; every FC1 and FC2 output element is
    compared.  `fc1_chunks`: precomputed oracle FC1 slices on the oracle's A1
    (the GPU's A1 is first checked to be bit-identical to it).  Returns y,
    the intermediates and the oracle FC2 slices on the GPU's A2."""
    y, it = _forward(w, W1, W2, align=align, fc1_out=True, y_rows_f32=True)
    ref = O.moe_permute(w.x, w.topk_idx, w.topk_prob, w.experts, align)
    off = it["expert_offsets"]
    assert np.array_equal(off, ref["offsets"])
    assert np.array_equal(it["dst_row"], ref["dst_row"])
    R = int(off[-1])
    assert np.array_equal(it["row_src"][:R], ref["row_src"][:R])
    assert np.array_equal(it["row_prob"][:R].view(np.uint32), ref["row_prob"][:R].view(np.uint32))
    for a, b in (("a1_codes", "codes"), ("a1_scales", "scales"), ("a1_gscale", "gscale")):
        assert np.array_equal(it[a][:R].view(np.uint8), ref[b][:R].view(np.uint8)), a
    A1 = (it["a1_codes"], it["a1_scales"], it["a1_gscale"])
    C = it["fc1_out"][:R]
    assert_gemm_full(C, A1, W1, off, "FC1", chunks=fc1_chunks)
    D = it["d"][:R]
    dref, _ = O.swiglu(C, it["row_prob"][:R])
    dv = bf16_bits_to_f32(D).astype(np.float64)
    rv = bf16_bits_to_f32(dref).astype(np.float64)
    assert np.all(np.abs(dv - rv) <= bf16_ulp(rv) * 1.0001 + 1e-40), "SwiGLU D"
    amax = it["amax_d"][:R]
    assert np.array_equal(amax, np.abs(bf16_bits_to_f32(D)).max(axis=1)), "amax_d"
    a2 = O.quantize(D, amax_in=amax)
    for name, r in zip(("a2_codes", "a2_scales", "a2_gscale"), a2):
        assert np.array_equal(it[name][:R].view(np.uint8), r.view(np.uint8)), name
    A2 = (it["a2_codes"], it["a2_scales"], it["a2_gscale"])
    Y = it["y_rows_f32"][:R]
    fc2_chunks = list(oracle_gemm_chunks(A2, W2, off))
    assert_gemm_full(Y, A2, W2, off, "FC2", chunks=fc2_chunks)
    # combine: y vs the oracle combine of the GPU's own rows
    ycomb = bf16_bits_to_f32(O.combine(Y, it["dst_row"])).astype(np.float64)
    yv = bf16_bits_to_f32(y).astype(np.float64)
    # fp32 accumulation of k terms + one bf16 rounding on each side
    absum = np.zeros_like(yv)
    dst = it["dst_row"]
    for j in range(dst.shape[1]):
        ok = dst[:, j] >= 0
        absum[ok] += np.abs(Y[dst[ok, j]])
    tol = absum * 2.0 ** -20 + bf16_ulp(ycomb) * 1.0001 + 1e-30
    assert np.all(np.abs(yv - ycomb) <= tol), "combine"
    return y, it, fc2_chunks


def _requant_flip_rate(it, ref, rows):
    """Fraction of FC2-input E2M1 codes (nibbles of the routed rows) that differ
    between the GPU layer and a pure oracle run.  They differ only where the
    two FC1 accumulations round a D value differently, which moves a code
    across a threshold or changes the row's amax."""
    g = it["a2_codes"][:rows].view(np.uint8)
    o = ref["a2_codes"][:rows].view(np.uint8)
    diff = ((g & 0xF) != (o & 0xF)).sum() + ((g >> 4) != (o >> 4)).sum()
    return diff / (2.0 * g.size)


@pytest.mark.parametrize("align", [1, 16])
def test_tiny_layer_replay_chain_and_end_to_end(align):
    w, W1, W2 = moe_case(0)
    y, it, _ = _replay_chain(w, W1, W2, align)
    yo, ref = O.moe_forward(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2, align=align)
    a = bf16_bits_to_f32(y).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    flips = _requant_flip_rate(it, ref, int(it["expert_offsets"][-1]))
    print(f"tiny layer end-to-end rel L2 vs pure oracle: {rel:.3e}, requant code flips {flips:.2e}")
    assert rel < 1e-2
    assert flips < 1e-2


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_workload_layer_replay_chain(wid):
    """The Qwen3-shaped, decode-shaped and long heavy-tail layers at full
    size: every FC1 and FC2 output element of every routed row."""
    w, W1, W2 = moe_case(wid)
    _replay_chain(w, W1, W2, 1, fc1_oracle_chunks(wid) if wid == 2 else None)


def test_decode_layer_end_to_end():
    w, W1, W2 = moe_case(3)
    y, it = _forward(w, W1, W2)
    yo, ref = O.moe_forward(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2)
    a = bf16_bits_to_f32(y).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    flips = _requant_flip_rate(it, ref, int(it["expert_offsets"][-1]))
    print(f"decode layer end-to-end rel L2 vs pure oracle: {rel:.3e}, requant code flips {flips:.2e}")
    assert rel < 1e-2
    assert flips < 1e-2


def test_perf_path_bf16_rows_and_determinism():
    """The benchmarked configuration (bf16 FC2 rows, no debug outputs) gives
    the same y on repeated calls, and its FC2 rows are the bf16 rounding of
    values within the GEMM tolerance."""
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_forward
    w, W1, W2 = moe_case(2)
    args = (dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts, w.inter, _weights(W1),
            _weights(W2))
    say("moe_expert_forward perf path x2")
    y1 = moe_expert_forward(*args)
    y2 = moe_expert_forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y, it = _forward(w, W1, W2)
    assert np.array_equal(y, host(y1))
    # static weights in the tiled layout: the same bits
    say("moe_expert_forward tiled weights")
    yt = moe_expert_forward(*args[:5], _weights(W1).packed(), _weights(W2).packed())
    torch.cuda.synchronize()
    assert torch.equal(yt, y1)
    # every bf16 FC2 row element of the timed path (tiled weights, bf16 rows):
    # the round-to-nearest-even of a value within the GEMM tolerance of the
    # oracle on the same A2
    yd, it = _forward(w, W1, W2, tiled=True)
    assert np.array_equal(yd, host(y1))
    A2 = (it["a2_codes"], it["a2_scales"], it["a2_gscale"])
    n = assert_gemm_full(it["y_rows"], A2, W2, it["expert_offsets"], "FC2 bf16 rows",
                         bf16_out=True)
    assert n == int(it["expert_offsets"][-1]) * w.hidden


def test_decode_perf_path_matches_the_checked_path():
    """The decode-shaped layer as the benchmark runs it (tiled weights, no
    debug outputs, the 32-row tile) gives the checked debug path's y bit for
    bit, on repeated calls."""
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_forward
    w, W1, W2 = moe_case(3)
    say("decode layer perf path x2")
    args = (dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts, w.inter,
            _weights(W1).packed(), _weights(W2).packed())
    y1 = moe_expert_forward(*args)
    y2 = moe_expert_forward(*args)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    y, _ = _forward(w, W1, W2)
    assert np.array_equal(y, host(y1))


@pytest.mark.parametrize("tokens,experts,zipf", [(160, 300, 0.0), (2000, 300, 1.2), (600, 1024, 0.0),
                                                (2200, 1024, 0.0), (16384, 128, 1.2), (16448, 128, 1.2)])
def test_many_experts_replay_chain(tokens, experts, zipf):
    """300 experts: the layer's precomputed tile schedules span groups held by
    several waves of their builder, on the 32-row tile (about 3 rows per
    expert) and on the 128-row tile with skewed routing (empty, tiny and
    multi-tile experts); 1024 experts, the largest count, fill every group
    slot of the builder; every step of the chain is checked in full.  At
    2200 tokens the chunk-count matrix (1024 x 35) is past what one
    workgroup of the fused scan-and-entries launch reads, so the routing
    takes its three-launch form; at 600 tokens (10 chunks, not a multiple of
    4) the fused launch sums the matrix element by element, each thread's
    stretch crossing several experts' rows.  16384 and 16448 tokens with 128
    experts sit on either side of the fused launch's limit (32768 and 32896
    matrix entries)."""
    from nvfp4_w4a4_quantized_amd.workloads import MoeWorkload, random_bf16, route_topk
    rng = np.random.default_rng(tokens + experts)
    H, I, k = 256, 128, 6
    logits = rng.standard_normal((tokens, experts)).astype(np.float32)
    if zipf:
        logits += (-zipf * np.log(np.arange(1, experts + 1))).astype(np.float32)
    idx, prob = route_topk(logits, k)
    w = MoeWorkload(f"many_experts_t{tokens}", -1, tokens, H, I, experts, k,
                    random_bf16(rng, (tokens, H)), idx, prob, None, None, {})
    from gpu_util import oracle_weights
    W1 = oracle_weights(random_bf16(rng, (experts, 2 * I, H), 0.02))
    W2 = oracle_weights(random_bf16(rng, (experts, H, I), 0.02))
    y, it, _ = _replay_chain(w, W1, W2, 1)
    yo, _ = O.moe_forward(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2)
    a = bf16_bits_to_f32(y).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-2


@pytest.mark.parametrize("tokens,experts,k", [(400, 64, 20), (700, 40, 12)])
def test_wide_topk_replay_chain(tokens, experts, k):
    """Top-k above 8 through the layer: the routing's generic histogram (no
    unrolled id list at k = 20), and at k = 20 chunks of 64 tokens holding
    1280 entries, so the fused scan-and-entries launch also places entries
    past the 1024 it preloads (4 per thread); k = 12 (768 per chunk) stays
    within them.  Every step of the chain in full."""
    from nvfp4_w4a4_quantized_amd.workloads import MoeWorkload, random_bf16, route_topk
    rng = np.random.default_rng(tokens + experts + k)
    H, I = 256, 128
    idx, prob = route_topk(rng.standard_normal((tokens, experts)).astype(np.float32), k)
    w = MoeWorkload(f"wide_topk_t{tokens}_k{k}", -1, tokens, H, I, experts, k,
                    random_bf16(rng, (tokens, H)), idx, prob, None, None, {})
    from gpu_util import oracle_weights
    W1 = oracle_weights(random_bf16(rng, (experts, 2 * I, H), 0.02))
    W2 = oracle_weights(random_bf16(rng, (experts, H, I), 0.02))
    y, it, _ = _replay_chain(w, W1, W2, 1)
    yo, _ = O.moe_forward(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2)
    a = bf16_bits_to_f32(y).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-2


@pytest.mark.parametrize("H,I", [(16384, 128), (256, 16384)])
def test_largest_hidden_and_intermediate_replay_chain(H, I):
    """The layer at its largest hidden size (FC1's K, FC2's N) and at its
    largest intermediate size (FC1's N, FC2's K): every step of the chain in
    full, and y against the oracle layer."""
    from nvfp4_w4a4_quantized_amd.workloads import MoeWorkload, random_bf16, route_topk
    rng = np.random.default_rng(H + I)
    tokens, experts, k = 96, 4, 2
    idx, prob = route_topk(rng.standard_normal((tokens, experts)).astype(np.float32), k)
    w = MoeWorkload(f"largest_h{H}_i{I}", -1, tokens, H, I, experts, k,
                    random_bf16(rng, (tokens, H)), idx, prob, None, None, {})
    from gpu_util import oracle_weights
    W1 = oracle_weights(random_bf16(rng, (experts, 2 * I, H), 0.02))
    W2 = oracle_weights(random_bf16(rng, (experts, H, I), 0.02))
    y, it, _ = _replay_chain(w, W1, W2, 1)
    yo, _ = O.moe_forward(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2)
    a = bf16_bits_to_f32(y).astype(np.float64)
    b = bf16_bits_to_f32(yo).astype(np.float64)
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-2


@pytest.mark.parametrize("tokens,align", [(0, 1), (0, 16), (1, 1), (1, 16)])
def test_empty_and_single_token_layer(tokens, align):
    """No tokens: the tile tables are empty and every GEMM workgroup exits;
    y is empty.  One token: k rows in k experts (padded rows with align > 1),
    checked against the oracle layer."""
    from nvfp4_w4a4_quantized_amd.ops import moe_expert_forward
    w, W1, W2 = moe_case(0)
    x, idx, prob = w.x[:tokens], w.topk_idx[:tokens], w.topk_prob[:tokens]
    say("moe_expert_forward tokens", tokens, "align", align)
    y = moe_expert_forward(dev_bf16(x.reshape(tokens, w.hidden)), dev(idx.reshape(tokens, w.topk)),
                           dev(prob.reshape(tokens, w.topk)), w.experts, w.inter, _weights(W1),
                           _weights(W2), align=align)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (tokens, w.hidden)
    if tokens:
        yo, _ = O.moe_forward(x, idx, prob, w.experts, w.inter, W1, W2, align=align)
        a = bf16_bits_to_f32(host(y)).astype(np.float64)
        b = bf16_bits_to_f32(yo).astype(np.float64)
        assert np.linalg.norm(a - b) <= 2e-2 * np.linalg.norm(b) + 1e-6


@pytest.mark.parametrize("wid", [0, 2, 3])
def test_forward_equals_composed_calls(wid):
    """moe_expert_forward (GEMM tiles from the tables its routing launch
    writes) against the same layer composed from the public calls (GEMM tiles
    from each workgroup's own lookup): every kernel is deterministic and an
    output element sees the same arithmetic whichever workgroup computes it,
    so y matches bit for bit."""
    from nvfp4_w4a4_quantized_amd import ops
    w, W1, W2 = moe_case(wid)
    x, idx, prob = dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob)
    w1, w2 = _weights(W1), _weights(W2)
    say("forward vs composed calls", wid)
    y = ops.moe_expert_forward(x, idx, prob, w.experts, w.inter, w1, w2)
    p = ops.moe_permute(x, idx, prob, w.experts)
    d, amax, _ = ops.w4a4_grouped_gemm_swiglu(p["codes"], p["scales"], p["gscale"], w1,
                                             p["offsets"], p["row_prob"])
    a2c, a2s, a2g = ops.nvfp4_quantize(d, amax_in=amax)
    rows = ops.w4a4_grouped_gemm(a2c, a2s, a2g, w2, p["offsets"], out_dtype=torch.bfloat16)
    yc = ops.moe_combine(rows, p["dst_row"])
    torch.cuda.synchronize()
    assert torch.equal(y, yc)
