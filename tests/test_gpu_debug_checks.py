"""The debug build (NVFP4_DEBUG_CHECKS) checks the data preconditions of the
routing on the device and reports them in the precondition word, the first
uint32 of the workspace: a token naming one expert twice (bit 0x1), a
non-finite activation (0x2), a non-finite router weight (0x4).  Clean inputs
leave the word 0 and give the release build's outputs bit for bit.  Violated
preconditions stay fault-free by construction (ranks of a duplicated id stay
inside the expert's counted rows; the quantizer has no value-dependent
control flow), so these inputs are safe to run."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, moe_case, say
from nvfp4_w4a4_quantized_amd import _lib
from nvfp4_w4a4_quantized_amd.workloads import random_bf16, route_topk

pytestmark = pytest.mark.gpu

DUP, BADX, BADP = 0x1, 0x2, 0x4


def _word(ws: torch.Tensor) -> int:
    torch.cuda.synchronize()
    return int(host(ws[:4]).view(np.uint32)[0])


def _case(tokens, experts, k, hidden, seed):
    rng = np.random.default_rng(seed)
    x = random_bf16(rng, (tokens, hidden))
    idx, prob = route_topk(rng.standard_normal((tokens, experts)).astype(np.float32), k)
    return x, idx, prob


def _permute(x, idx, prob, E, library):
    from nvfp4_w4a4_quantized_amd import ops
    T, k = idx.shape
    wsb = int(library.moe_permute_workspace_size(T, k, E))
    ws = torch.full((wsb,), 0xAB, dtype=torch.uint8, device="cuda")
    out = ops.moe_permute(dev_bf16(x) if x is not None else None, dev(idx), dev(prob), E,
                          workspace=ws, library=library)
    return out, ws


# (tokens, experts, topk, hidden): the one-launch small-batch path, the
# three-launch path, and top-k above 16 (ids resolved entry by entry)
SHAPES = [(256, 16, 4, 256), (1100, 64, 8, 512), (300, 64, 20, 128)]


@pytest.mark.parametrize("shape", SHAPES, ids=["small", "large", "wide_topk"])
def test_clean_inputs_word_zero_and_release_bits(shape):
    T, E, k, H = shape
    x, idx, prob = _case(T, E, k, H, T + E)
    say("debug checks: clean", shape)
    rel, _ = _permute(x, idx, prob, E, _lib.lib())
    dbg, ws = _permute(x, idx, prob, E, _lib.debug_lib())
    assert _word(ws) == 0
    R = int(host(rel["offsets"])[-1])
    for name in ("offsets", "dst_row"):
        assert torch.equal(rel[name], dbg[name]), name
    for name in ("row_src", "row_prob", "codes", "scales", "gscale"):
        assert torch.equal(rel[name][:R], dbg[name][:R]), name


@pytest.mark.parametrize("shape", SHAPES, ids=["small", "large", "wide_topk"])
def test_each_violation_sets_its_bit(shape):
    T, E, k, H = shape
    x, idx, prob = _case(T, E, k, H, 7 * T + E)
    L = _lib.debug_lib()
    # a token naming one expert twice (the second entry overwritten)
    i2 = idx.copy()
    i2[T // 2, 1] = i2[T // 2, 0]
    say("debug checks: duplicate id", shape)
    _, ws = _permute(x, i2, prob, E, L)
    assert _word(ws) == DUP
    # ids outside [0, E) are "not routed", not a violation, even when repeated
    i3 = idx.copy()
    i3[3, 0] = i3[3, 1] = -1
    i3[4, 0] = i3[4, 1] = E + 5
    say("debug checks: dropped ids", shape)
    _, ws = _permute(x, i3, prob, E, L)
    assert _word(ws) == 0
    # a NaN and an Inf activation in two tokens
    x2 = x.copy()
    x2[T - 1, H - 1] = 0x7FC0
    x2[1, 3] = 0xFF80
    say("debug checks: non-finite x", shape)
    _, ws = _permute(x2, idx, prob, E, L)
    assert _word(ws) == BADX
    # metadata only: x is not read, so no activation is checked
    say("debug checks: metadata only", shape)
    _, ws = _permute(None, idx, prob, E, L)
    assert _word(ws) == 0
    # a non-finite router weight, together with a duplicate
    p2 = prob.copy()
    p2[0, k - 1] = np.inf
    say("debug checks: inf prob + duplicate", shape)
    _, ws = _permute(x, i2, p2, E, L)
    assert _word(ws) == DUP | BADP
    # the word is cleared by each call
    say("debug checks: clean after dirty", shape)
    _, ws2 = _permute(x, idx, prob, E, L)
    assert _word(ws2) == 0


def test_layer_reports_in_its_workspace():
    """moe_expert_forward's workspace carries the same word (byte offset 0)."""
    from nvfp4_w4a4_quantized_amd import ops
    w, W1, W2 = moe_case(0)
    L = _lib.debug_lib()
    w1 = ops.NvFp4Weights(dev(W1[0]), dev(W1[1]), dev(W1[2]))
    w2 = ops.NvFp4Weights(dev(W2[0]), dev(W2[1]), dev(W2[2]))
    wsb = int(L.moe_expert_forward_workspace_size(w.tokens, w.hidden, w.inter, w.topk,
                                                  w.experts, 1))
    idx = w.topk_idx.copy()
    idx[10, 1] = idx[10, 0]
    for ids, want in ((w.topk_idx, 0), (idx, DUP)):
        ws = torch.zeros(wsb, dtype=torch.uint8, device="cuda")
        say("debug checks: layer", want)
        y = ops.moe_expert_forward(dev_bf16(w.x), dev(ids), dev(w.topk_prob), w.experts, w.inter,
                                   w1, w2, workspace=ws, library=L)
        assert _word(ws) == want
        if want == 0:
            yr = ops.moe_expert_forward(dev_bf16(w.x), dev(ids), dev(w.topk_prob), w.experts,
                                        w.inter, w1, w2)
            torch.cuda.synchronize()
            assert torch.equal(y, yr)
