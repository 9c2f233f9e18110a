"""moe_permute_noalloc (the entry point that allocates nothing; its routing
scratch is the library's static device array) against moe_permute with a
caller workspace, through the C ABI: every output bit-identical, on calls in
a row whose later inputs are smaller (the array keeps the previous call's
contents), on the three-launch path, the one-launch small-batch path, with
padding and metadata only."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, say
from nvfp4_w4a4_quantized_amd.workloads import random_bf16, route_topk

pytestmark = pytest.mark.gpu


def _inputs(tokens, experts, k, hidden, seed, zipf=0.0):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((tokens, experts)).astype(np.float32)
    if zipf:
        logits += (-zipf * np.log(np.arange(1, experts + 1))).astype(np.float32)
    idx, prob = route_topk(logits, k)
    x = random_bf16(rng, (tokens, hidden))
    return dev_bf16(x), dev(idx), dev(prob)


def _compare(ref, got, what):
    R = int(host(ref["offsets"])[-1])
    assert torch.equal(ref["offsets"], got["offsets"]), what
    assert torch.equal(ref["dst_row"], got["dst_row"]), what
    for name in ("row_src", "row_prob", "codes", "scales", "gscale"):
        if name in ref:
            assert torch.equal(ref[name][:R], got[name][:R]), f"{what}: {name}"


# (tokens, experts, topk, hidden, align, zipf): largest first, each later
# call smaller than the one before
CALLS = [
    (32768, 128, 8, 2048, 1, 1.3),   # the long-sequence layer: 512 KiB of scratch
    (8192, 128, 8, 2048, 16, 1.1),   # Qwen3-shaped routing, padded to 16 rows
    (1100, 64, 8, 512, 1, 0.0),
    (300, 16, 4, 256, 1, 0.0),       # one-launch small-batch path
]


@pytest.mark.parametrize("order", ["descending", "repeat_small_after_large"])
def test_noalloc_matches_workspace_entry_point(order):
    from nvfp4_w4a4_quantized_amd import ops
    calls = CALLS if order == "descending" else [CALLS[0], CALLS[3], CALLS[1], CALLS[3]]
    for i, (T, E, k, H, align, zipf) in enumerate(calls):
        x, idx, prob = _inputs(T, E, k, H, 100 + i, zipf)
        say("noalloc permute", order, i, (T, E, k, H, align))
        got = ops.moe_permute_noalloc(x, idx, prob, E, align=align)
        ref = ops.moe_permute(x, idx, prob, E, align=align)
        torch.cuda.synchronize()
        _compare(ref, got, f"call {i} {(T, E, k, H, align)}")


def test_noalloc_metadata_only_and_outputs_reused():
    """x = NULL (metadata only), then two calls into the same output buffers
    (the caller-owned outputs are the only memory the call touches besides
    the static scratch)."""
    from nvfp4_w4a4_quantized_amd import ops
    x, idx, prob = _inputs(4096, 128, 8, 2048, 7, 1.1)
    say("noalloc permute metadata only")
    got = ops.moe_permute_noalloc(None, idx, prob, 128)
    ref = ops.moe_permute(None, idx, prob, 128)
    torch.cuda.synchronize()
    _compare(ref, got, "metadata only")
    out = ops.moe_permute_noalloc(x, idx, prob, 128)
    for seed in (8, 9):
        x2, idx2, prob2 = _inputs(4096, 128, 8, 2048, seed, 1.1)
        say("noalloc permute into reused outputs", seed)
        got = ops.moe_permute_noalloc(x2, idx2, prob2, 128, out=out)
        ref = ops.moe_permute(x2, idx2, prob2, 128)
        torch.cuda.synchronize()
        _compare(ref, got, f"reused outputs {seed}")
