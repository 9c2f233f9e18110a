"""GPU parity of moe_permute (through the C ABI) against the oracle: expert
offsets, dst_row, row_src, row_prob and the quantized rows must match bit for
bit, including padding rows, empty experts and dropped entries."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, moe_case, say
from nvfp4_w4a4_quantized_amd.workloads import random_bf16
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _permute_and_compare(x, idx, prob, E, align, what):
    from nvfp4_w4a4_quantized_amd.ops import moe_permute
    say("moe_permute", what, "T", idx.shape[0], "k", idx.shape[1], "E", E, "align", align)
    out = moe_permute(None if x is None else dev_bf16(x), dev(idx), dev(prob), E, align)
    torch.cuda.synchronize()
    ref = O.moe_permute(x, idx, prob, E, align)
    off = host(out["offsets"])
    assert np.array_equal(off, ref["offsets"]), f"{what}: offsets"
    assert np.array_equal(host(out["dst_row"]), ref["dst_row"]), f"{what}: dst_row"
    R = int(off[-1])
    assert np.array_equal(host(out["row_src"])[:R], ref["row_src"][:R]), f"{what}: row_src"
    assert np.array_equal(host(out["row_prob"])[:R].view(np.uint32),
                          ref["row_prob"][:R].view(np.uint32)), f"{what}: row_prob"
    if x is not None:
        assert np.array_equal(host(out["gscale"])[:R].view(np.uint32),
                              ref["gscale"][:R].view(np.uint32)), f"{what}: gscale"
        assert np.array_equal(host(out["scales"])[:R], ref["scales"][:R]), f"{what}: scales"
        assert np.array_equal(host(out["codes"])[:R], ref["codes"][:R]), f"{what}: codes"
    return out, ref


@pytest.mark.parametrize("wid", [0, 2, 3, 4])
def test_workload_routing(wid):
    w, _, _ = moe_case(wid, with_weights=False)
    _permute_and_compare(w.x, w.topk_idx, w.topk_prob, w.experts, 1, f"workload {wid}")


@pytest.mark.parametrize("align", [1, 16, 128])
def test_alignment_padding(align):
    w, _, _ = moe_case(0, with_weights=False)
    _permute_and_compare(w.x, w.topk_idx, w.topk_prob, w.experts, align, f"tiny align {align}")


def _fixture_routing(rng, T, k, E, kind):
    if kind == "empty_and_tiny":
        # experts 0..3 get exactly 0, 1, 2, 3 rows; the rest random among 8..E-1
        idx = np.zeros((T, k), np.int32)
        for t in range(T):
            idx[t] = rng.choice(np.arange(8, E), size=k, replace=False)
        forced = [(1, 1), (2, 2), (3, 3), (4, 1)]    # (expert, rows)
        t = 0
        for e, n in forced:
            for _ in range(n):
                if t < T:
                    idx[t, 0] = e
                t += 1
        return idx
    if kind == "one_expert":
        idx = np.zeros((T, k), np.int32)
        for t in range(T):
            idx[t] = np.concatenate([[5], rng.choice(np.delete(np.arange(E), 5), size=k - 1, replace=False)])
        return idx
    if kind == "dropped":
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        mask = rng.random((T, k)) < 0.2
        idx[mask] = np.where(rng.random(mask.sum()) < 0.5, -1, E + 3)
        return idx
    raise ValueError(kind)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 300, 1024, 1025, 1100])
@pytest.mark.parametrize("kind", ["empty_and_tiny", "one_expert", "dropped"])
def test_edge_routings(T, kind):
    """Up to 4096 routing entries (T*k) the permutation runs as one launch
    that histograms the ids in every workgroup (T = 1024: exactly 4096, every
    thread holding 16 of them); from T = 1025 (4100 entries) it takes the
    histogram / scan / scatter launches."""
    rng = np.random.default_rng(T * 31 + len(kind))
    E, k, H = 16, 4, 256
    idx = _fixture_routing(rng, T, k, E, kind)
    prob = rng.random((T, k)).astype(np.float32)
    x = random_bf16(rng, (T, H))
    x[0] = 0x8000                              # a -0.0 row
    for align in (1, 16):
        _permute_and_compare(x, idx, prob, E, align, f"{kind} T={T}")


@pytest.mark.parametrize("T", [1000, 300])
def test_metadata_only_and_many_experts(T):
    """1024 experts, on both permutation paths (8000 and 2400 entries)."""
    rng = np.random.default_rng(3 + T)
    k, E = 8, 1024
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    prob = rng.random((T, k)).astype(np.float32)
    _permute_and_compare(None, idx, prob, E, 1, "metadata only E=1024")
    x = random_bf16(rng, (T, 128))
    _permute_and_compare(x, idx, prob, E, 4, "E=1024 H=128")


def test_zero_tokens():
    from nvfp4_w4a4_quantized_amd.ops import moe_permute
    idx = np.zeros((0, 2), np.int32)
    prob = np.zeros((0, 2), np.float32)
    say("moe_permute T=0")
    out = moe_permute(dev_bf16(np.zeros((0, 64), np.uint16)), dev(idx), dev(prob), 4, 16)
    torch.cuda.synchronize()
    assert host(out["offsets"]).tolist() == [0, 0, 0, 0, 0]


def test_deterministic_repeat():
    w, _, _ = moe_case(2, with_weights=False)
    from nvfp4_w4a4_quantized_amd.ops import moe_permute
    a = moe_permute(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts)
    b = moe_permute(dev_bf16(w.x), dev(w.topk_idx), dev(w.topk_prob), w.experts)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("k,E", [(12, 40), (20, 64)])
@pytest.mark.parametrize("T", [200, 400])
def test_wide_topk(k, E, T):
    """top-k beyond 8 (16-id register path) and beyond 16 (generic path), on
    the one-launch permutation (T = 200) and the three-launch one (T = 400)."""
    rng = np.random.default_rng(k + T)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    idx[3, 2] = -1
    prob = rng.random((T, k)).astype(np.float32)
    x = random_bf16(rng, (T, 128))
    for align in (1, 8):
        _permute_and_compare(x, idx, prob, E, align, f"k={k} E={E}")
