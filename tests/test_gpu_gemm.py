"""GPU parity of the W4A4 grouped GEMM and its fused SwiGLU epilogue (through
the C ABI) against the oracle, within |gpu - oracle| <= 2^-10 * sum|a_k b_k|
+ 1e-6 (fp32 output).  Every case compares every output element, the
full-size workloads included (the oracle's result and bound are computed in
row slices)."""
import numpy as np
import pytest
import torch

from gpu_util import (assert_gemm_close, assert_gemm_full, bf16_ulp, dev, dev_bf16,
                      fc1_oracle_chunks, host, moe_case, moe_permute_ref, oracle_weights, say)
from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, make_dense, random_bf16
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def _weights(W, tiled=False):
    from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights
    w = NvFp4Weights(dev(W[0]), dev(W[1]), dev(W[2]))
    return w.packed() if tiled else w


def _operands(rng, rows, G, n, k, scale=1.0):
    a = random_bf16(rng, (rows, k), scale)
    A = O.quantize(a)
    W = oracle_weights(random_bf16(rng, (G, n, k), 0.02))
    return A, W


def _run_plain(A, W, offs, dtype=torch.float32, tiled=False):
    from nvfp4_w4a4_quantized_amd.ops import w4a4_grouped_gemm
    out = w4a4_grouped_gemm(dev(A[0]), dev(A[1]), dev(A[2]), _weights(W, tiled), dev(offs),
                            out_dtype=dtype)
    torch.cuda.synchronize()
    return host(out) if dtype == torch.float32 else bf16_bits_to_f32(host(out))


@pytest.mark.parametrize("shape", [
    # rows, offsets, n, k
    (300, [0, 300], 256, 256),
    (300, [0, 1, 2, 5, 9, 9, 130, 300], 96, 128),       # tiny and empty groups, n % 128 != 0
    (513, [0, 200, 200, 513], 160, 768),
    (257, [3, 100, 257], 2048, 384),                     # rows before off[0] untouched
    (64, [0, 64], 32, 2048),
    (160, [0, 70, 160], 64, 16384),                      # the largest K, 128-row tile
    (40, [0, 9, 40], 96, 16384),                          # the largest K, 32-row tile
])
def test_plain_fp32_full_compare(shape):
    rows, offs, n, k = shape
    offs = np.array(offs, np.int32)
    G = offs.size - 1
    rng = np.random.default_rng(rows + n + k)
    A, W = _operands(rng, rows, G, n, k)
    say("gemm fp32", rows, offs.tolist(), n, k)
    gpu = _run_plain(A, W, offs)
    ref, bound = O.grouped_gemm(*A, *W, offs, with_bound=True)
    r0, r1 = offs[0], offs[-1]
    assert_gemm_close(gpu[r0:r1], ref[r0:r1], bound[r0:r1], f"plain {shape}")
    # the tiled weight layout computes the same bits
    say("gemm fp32 tiled B", rows, offs.tolist(), n, k)
    gpu_t = _run_plain(A, W, offs, tiled=True)
    assert np.array_equal(gpu_t[r0:r1].view(np.uint32), gpu[r0:r1].view(np.uint32))


def test_many_groups_full_compare():
    """More groups than one 256-group chunk of the tile schedule, with empty,
    tiny and multi-tile groups (every tile assigned once)."""
    rng = np.random.default_rng(17)
    G, n, k = 300, 64, 128
    sizes = rng.integers(0, 12, G)
    sizes[rng.integers(0, G, 5)] = [0, 129, 300, 1, 255]
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offs[-1])
    A, W = _operands(rng, rows, G, n, k)
    say("gemm many groups", G, rows, n, k)
    gpu = _run_plain(A, W, offs)
    ref, bound = O.grouped_gemm(*A, *W, offs, with_bound=True)
    assert_gemm_close(gpu, ref, bound, "many groups")


def test_pack_weights_is_the_documented_permutation():
    """nvfp4_pack_weights against the byte map stated in the header, written
    out here with numpy index arithmetic."""
    rng = np.random.default_rng(21)
    G, n, k = 3, 96, 384
    codes = rng.integers(0, 256, (G, n, k // 2)).astype(np.uint8)
    scales = rng.integers(0, 256, (G, n, k // 16)).astype(np.uint8)
    say("pack weights", G, n, k)
    w = _weights((codes, scales, np.ones(G, np.float32)), tiled=True)
    torch.cuda.synchronize()
    pc, ps = host(w.codes).reshape(-1), host(w.scales).reshape(-1)
    nst, nrb = k // 128, n // 32
    exp_c = np.empty(G * n * k // 2, np.uint8)
    exp_s = np.empty(G * n * k // 16, np.uint8)
    for g in range(G):
        for rb in range(nrb):
            for st in range(nst):
                t = (g * nrb + rb) * nst + st
                for L in range(64):
                    row = 32 * rb + L % 32
                    for c in range(2):
                        src = 64 * st + 32 * (L // 32) + 16 * c
                        dst = t * 2048 + c * 1024 + 16 * L
                        exp_c[dst:dst + 16] = codes[g, row, src:src + 16]
                    src = 8 * st + 4 * (L // 32)
                    exp_s[t * 256 + 4 * L:t * 256 + 4 * L + 4] = scales[g, row, src:src + 4]
    assert np.array_equal(pc, exp_c)
    assert np.array_equal(ps, exp_s)


def test_plain_bf16_output():
    rng = np.random.default_rng(5)
    offs = np.array([0, 40, 41, 200], np.int32)
    A, W = _operands(rng, 200, 3, 256, 512)
    say("gemm bf16 out")
    gpu = _run_plain(A, W, offs, torch.bfloat16)
    ref, bound = O.grouped_gemm(*A, *W, offs, with_bound=True)
    # bf16 rounding of a value within the fp32 tolerance
    err = np.abs(gpu.astype(np.float64) - ref)
    assert np.all(err <= 2.0 ** -10 * bound + 1e-6 + bf16_ulp(ref) * 0.5 * 1.0001)


def test_one_hot_rows_are_exact():
    k, n = 128, 64
    a_codes = np.zeros((k, k // 2), np.uint8)
    for i in range(k):
        a_codes[i, i // 2] = 7 << (4 * (i % 2))
    a_scales = np.full((k, k // 16), 0x38, np.uint8)
    a_g = np.full(k, 0.5, np.float32)
    rng = np.random.default_rng(6)
    W = (rng.integers(0, 256, (1, n, k // 2)).astype(np.uint8),
         rng.integers(0x08, 0x7F, (1, n, k // 16)).astype(np.uint8), np.array([0.25], np.float32))
    say("gemm one-hot")
    gpu = _run_plain((a_codes, a_scales, a_g), W, np.array([0, k], np.int32))
    ref = O.grouped_gemm(a_codes, a_scales, a_g, *W, np.array([0, k], np.int32))
    assert np.array_equal(gpu, ref)


def test_dense_attention_projections_full():
    """QKV (K=2048, N=5120) and O-proj (K=4096, N=2048) over 8192 tokens with
    outlier channels: every output element."""
    d = make_dense()
    for pname, x, w in d.projections:
        A = O.quantize(x)
        W = oracle_weights(w[None])
        offs = np.array([0, x.shape[0]], np.int32)
        say("dense gemm", pname, x.shape, w.shape)
        gpu = _run_plain(A, W, offs)
        n = assert_gemm_full(gpu, A, W, offs, f"dense {pname}")
        assert n == x.shape[0] * w.shape[0]


@pytest.mark.parametrize("wid", [2, 3])
def test_moe_fc1_fc2_shapes_full(wid):
    """FC1 (N=1536, K=2048) and FC2 (N=2048, K=768) over the workload's
    routing, on oracle-quantized operands, plain fp32 epilogue: every
    element of every routed row (group-boundary rows included)."""
    w, W1, W2 = moe_case(wid)
    p = moe_permute_ref(wid)
    offs = p["offsets"]
    A1 = (p["codes"], p["scales"], p["gscale"])
    rng = np.random.default_rng(12 + wid)
    say("moe fc1 plain", wid)
    gpu = _run_plain(A1, W1, offs, tiled=(wid == 2))
    assert_gemm_full(gpu, A1, W1, offs, f"FC1 workload {wid}", chunks=fc1_oracle_chunks(wid))
    # FC2 on oracle-quantized synthetic activations of the FC2 input shape
    R = offs[-1]
    dx = random_bf16(rng, (R, w.inter), 0.05)
    A2 = O.quantize(dx)
    say("moe fc2 plain", wid)
    gpu2 = _run_plain(A2, W2, offs, tiled=(wid == 2))
    assert_gemm_full(gpu2, A2, W2, offs, f"FC2 workload {wid}")


def _swiglu_case(A, W, offs, prob, what, tiled=False):
    from nvfp4_w4a4_quantized_amd.ops import w4a4_grouped_gemm_swiglu
    say("gemm swiglu", what, "tiled" if tiled else "")
    d, amax, c = w4a4_grouped_gemm_swiglu(dev(A[0]), dev(A[1]), dev(A[2]), _weights(W, tiled),
                                          dev(offs), dev(prob), with_c=True)
    torch.cuda.synchronize()
    r0, r1 = int(offs[0]), int(offs[-1])
    c = host(c)[r0:r1]
    d = host(d)[r0:r1]
    amax = host(amax)[r0:r1]
    return c, d, amax


def test_swiglu_epilogue_full_compare():
    rng = np.random.default_rng(13)
    rows, G, I, K = 400, 5, 128, 256
    offs = np.array([0, 0, 37, 38, 250, 400], np.int32)
    A, W = _operands(rng, rows, G, 2 * I, K, 4.0)
    prob = rng.random(rows).astype(np.float32)
    prob[5] = 0.0
    c, d, amax = _swiglu_case(A, W, offs, prob, "small")
    ref, bound = O.grouped_gemm(*A, *W, offs, with_bound=True)
    assert_gemm_close(c, ref, bound, "swiglu C")
    # D within one bf16 ulp of the oracle's SwiGLU applied to the GPU's C
    dref, _ = O.swiglu(c, prob)
    dv = bf16_bits_to_f32(d).astype(np.float64)
    rv = bf16_bits_to_f32(dref).astype(np.float64)
    assert np.all(np.abs(dv - rv) <= bf16_ulp(rv) * 1.0001 + 1e-40)
    # amax is exactly the max |D| of the GPU's own D
    assert np.array_equal(amax, np.abs(bf16_bits_to_f32(d)).max(axis=1))
    # the tiled weight layout computes the same bits
    ct, dt, at = _swiglu_case(A, W, offs, prob, "small", tiled=True)
    assert np.array_equal(ct.view(np.uint32), c.view(np.uint32))
    assert np.array_equal(dt, d) and np.array_equal(at.view(np.uint32), amax.view(np.uint32))


@pytest.mark.parametrize("wid", [0, 2])
def test_swiglu_workload(wid):
    w, W1, _ = moe_case(wid)
    p = moe_permute_ref(wid)
    offs = p["offsets"]
    A1 = (p["codes"], p["scales"], p["gscale"])
    c, d, amax = _swiglu_case(A1, W1, offs, p["row_prob"], f"workload {wid}")
    R = c.shape[0]
    assert_gemm_full(c, A1, W1, offs, "swiglu C", chunks=fc1_oracle_chunks(wid))
    dref, _ = O.swiglu(c, p["row_prob"][:R])
    dv = bf16_bits_to_f32(d).astype(np.float64)
    rv = bf16_bits_to_f32(dref).astype(np.float64)
    assert np.all(np.abs(dv - rv) <= bf16_ulp(rv) * 1.0001 + 1e-40)
    assert np.array_equal(amax, np.abs(bf16_bits_to_f32(d)).max(axis=1))


def _pad_rows(a: np.ndarray, rows: int) -> np.ndarray:
    """`a` with junk rows appended up to `rows` (the kernel never reads them
    for the groups' outputs; a larger row capacity selects the 128-row tile)."""
    fill = 0x5A if a.dtype == np.uint8 else 0.75
    return np.concatenate([a, np.full((rows - a.shape[0],) + a.shape[1:], fill, a.dtype)])


@pytest.mark.parametrize("epi", ["f32", "bf16", "swiglu"])
@pytest.mark.parametrize("tiled", [False, True])
@pytest.mark.parametrize("K", [384, 512])
def test_small_and_large_tiles_agree(epi, tiled, K):
    """Groups of a few rows (at most 32 on average) run on the 32 x 128 tile;
    the same problem with its row capacity padded past 32 rows per group runs
    on the 128-row tile (128 x 256; 128 x 512 with the SwiGLU epilogue).  Both
    match the oracle, and each other bit for bit
    (every output element sees the same MFMA sequence).  K = 384 (3 stages)
    takes the small tile's one-B-set loop, K = 512 (4 stages) its two-set
    loop."""
    rng = np.random.default_rng(31 + K)
    G = 24
    n = 256 if epi == "swiglu" else 160
    sizes = rng.integers(0, 24, G)
    sizes[[2, 7, 11]] = [0, 70, 33]            # empty, three 32-row blocks, a ragged second block
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offs[-1])
    assert R <= 32 * G
    A, W = _operands(rng, R, G, n, K, 2.0)
    prob = rng.random(R).astype(np.float32)
    big = 32 * G + 1
    Ab = tuple(_pad_rows(x, big) for x in A)
    outs = []
    for tag, AA in (("small tile", A), ("large tile", Ab)):
        say("gemm tiles", epi, "tiled" if tiled else "row-major", tag)
        if epi == "swiglu":
            pp = np.concatenate([prob, np.zeros(AA[0].shape[0] - R, np.float32)])
            c, d, amax = _swiglu_case(AA, W, offs, pp, tag, tiled)
            outs.append((c[:R], d[:R], amax[:R]))
        else:
            dt = torch.float32 if epi == "f32" else torch.bfloat16
            outs.append(_run_plain(AA, W, offs, dt, tiled)[:R])
    ref, bound = O.grouped_gemm(*A, *W, offs, with_bound=True)
    if epi == "swiglu":
        (c0, d0, m0), (c1, d1, m1) = outs
        assert_gemm_close(c0, ref, bound, "swiglu C, small tile")
        dref, _ = O.swiglu(c0, prob)
        dv = bf16_bits_to_f32(d0).astype(np.float64)
        rv = bf16_bits_to_f32(dref).astype(np.float64)
        assert np.all(np.abs(dv - rv) <= bf16_ulp(rv) * 1.0001 + 1e-40)
        assert np.array_equal(m0, np.abs(bf16_bits_to_f32(d0)).max(axis=1))
        assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))
        assert np.array_equal(d0, d1) and np.array_equal(m0.view(np.uint32), m1.view(np.uint32))
    else:
        g0, g1 = outs
        if epi == "f32":
            assert_gemm_close(g0, ref, bound, f"{epi}, small tile")
        else:
            err = np.abs(g0.astype(np.float64) - ref)
            assert np.all(err <= 2.0 ** -10 * bound + 1e-6 + bf16_ulp(ref) * 0.5 * 1.0001)
        assert np.array_equal(g0.view(np.uint32), g1.view(np.uint32))


def test_bf16_output_stays_inside_its_columns():
    """bf16 output with N % 64 == 32 (the last wave's second 32-column block
    lies past N) on both tiles: columns >= N of a wider output view and the
    rows after the buffer stay untouched."""
    from nvfp4_w4a4_quantized_amd.ops import w4a4_grouped_gemm
    rng = np.random.default_rng(33)
    n, K = 96, 256
    for offs, G in ((np.array([0, 70, 150], np.int32), 2),
                    (np.array([0, 5, 9, 30, 31, 40], np.int32), 5)):
        R = int(offs[-1])
        A, W = _operands(rng, R, G, n, K)
        say("gemm bf16 guard", n, offs.tolist())
        # rows R..R+7 of a sentinel buffer follow the output
        buf = torch.full(((R + 8) * n,), -7.0, dtype=torch.bfloat16, device="cuda")
        out = buf[:R * n].view(R, n)
        w4a4_grouped_gemm(dev(A[0]), dev(A[1]), dev(A[2]), _weights(W), dev(offs),
                          out_dtype=torch.bfloat16, out=out)
        torch.cuda.synchronize()
        tail = host(buf[R * n:])
        assert np.all(bf16_bits_to_f32(tail) == -7.0)
        ref, bound = O.grouped_gemm(*A, *W, offs, with_bound=True)
        got = bf16_bits_to_f32(host(out))
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= 2.0 ** -10 * bound + 1e-6 + bf16_ulp(ref) * 0.5 * 1.0001)
