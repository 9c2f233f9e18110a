"""Pins of the oracle's routing permutation, grouped GEMM, SwiGLU and combine
against library routines (numpy stable argsort / bincount / float64 matmul,
torch's fp64 silu), exact rational brute force and closed forms."""
import json
import os
from fractions import Fraction

import numpy as np
import torch

from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, make_moe, to_bf16_bits
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLD, "e2m1_grid.json")) as _f:
    GRID = np.array(json.load(_f)["magnitudes"], np.float64)
E4M3_VALUES = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def decode(codes, scales, gscale_rows):
    codes = np.asarray(codes)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    q = GRID[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sb = np.repeat(E4M3_VALUES[np.asarray(scales)], 16, axis=1)
    return q * sb * np.asarray(gscale_rows, np.float64)[:, None]


# ---------------------------------------------------------------- routing --

def _numpy_route(idx, prob, E, align):
    T, k = idx.shape
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    padded = (counts + align - 1) // align * align
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    order = np.argsort(np.where(valid, flat, E), kind="stable")     # stable by flat index
    dst = np.full(T * k, -1, np.int64)
    pos = 0
    for e in range(E):
        ent = order[pos:pos + counts[e]]
        dst[ent] = offsets[e] + np.arange(counts[e])
        pos += counts[e]
    return offsets, dst.reshape(T, k), counts


def test_route_matches_numpy_stable_sort():
    rng = np.random.default_rng(20)
    for (T, k, E, align) in [(64, 2, 4, 1), (300, 8, 128, 1), (257, 8, 16, 16), (100, 4, 7, 128)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        prob = rng.random((T, k)).astype(np.float32)
        off, dst, src, rp = O.route(idx, prob, E, align)
        off_n, dst_n, counts = _numpy_route(idx, prob, E, align)
        assert np.array_equal(off, off_n)
        assert np.array_equal(dst, dst_n)
        for t in range(T):
            for j in range(k):
                assert src[dst[t, j]] == t and rp[dst[t, j]] == prob[t, j]
        for e in range(E):
            pad = np.arange(off[e] + counts[e], off[e + 1])
            assert np.all(src[pad] == -1) and np.all(rp[pad] == 0)
            # ascending token inside the expert
            seg = src[off[e]:off[e] + counts[e]]
            assert np.all(np.diff(seg) > 0)


def test_route_dropped_ids_and_empty_experts():
    idx = np.array([[0, -1], [5, 0], [0, 2], [9, 2]], np.int32)     # E=4: -1, 5, 9 dropped
    prob = np.ones((4, 2), np.float32)
    off, dst, src, rp = O.route(idx, prob, 4, 1)
    assert off.tolist() == [0, 3, 3, 5, 5]
    assert dst.tolist() == [[0, -1], [-1, 1], [2, 3], [-1, 4]]
    assert src[:5].tolist() == [0, 1, 2, 2, 3]


def test_permute_rows_are_per_token_quantized_copies():
    w = make_moe(0, with_weights=False)
    p = O.moe_permute(w.x, w.topk_idx, w.topk_prob, w.experts, align=16)
    c, s, g = O.quantize(w.x)
    off, src = p["offsets"], p["row_src"]
    rows = off[-1]
    real = src[:rows] >= 0
    assert np.array_equal(p["codes"][:rows][real], c[src[:rows][real]])
    assert np.array_equal(p["scales"][:rows][real], s[src[:rows][real]])
    assert np.array_equal(p["gscale"][:rows][real], g[src[:rows][real]])
    assert np.all(p["codes"][:rows][~real] == 0) and np.all(p["gscale"][:rows][~real] == 0)


# ------------------------------------------------------------------- GEMM --

def _random_operands(rng, rows, G, n, k):
    a = to_bf16_bits(rng.standard_normal((rows, k)).astype(np.float32))
    b = to_bf16_bits((rng.standard_normal((G * n, k)) * 0.02).astype(np.float32))
    ac, as_, ag = O.quantize(a)
    boffs = np.arange(G + 1, dtype=np.int32) * n
    bc, bs, bg = O.quantize(b, domain=1, group_offsets=boffs)
    return (ac, as_, ag), (bc.reshape(G, n, k // 2), bs.reshape(G, n, k // 16), bg)


def test_gemm_matches_numpy_matmul_of_dequantized_operands():
    rng = np.random.default_rng(21)
    rows, G, n, k = 70, 3, 48, 256
    A, B = _random_operands(rng, rows, G, n, k)
    offs = np.array([0, 20, 20, 70], np.int32)
    out, bound = O.grouped_gemm(*A, *B, offs, with_bound=True)
    a_dq = decode(A[0], A[1], A[2])
    for g in range(G):
        r0, r1 = offs[g], offs[g + 1]
        if r1 == r0:
            continue
        b_dq = decode(B[0][g], B[1][g], np.full(n, B[2][g]))
        ref = a_dq[r0:r1] @ b_dq.T
        absref = np.abs(a_dq[r0:r1]) @ np.abs(b_dq).T
        assert np.all(np.abs(out[r0:r1] - ref) <= 2.0 ** -23 * np.abs(ref) + 1e-30)
        assert np.allclose(bound[r0:r1], absref, rtol=1e-12, atol=0)


def test_gemm_exact_rational_brute_force_tiny():
    rng = np.random.default_rng(22)
    rows, G, n, k = 5, 2, 3, 32
    A, B = _random_operands(rng, rows, G, n, k)
    offs = np.array([0, 2, 5], np.int32)
    out = O.grouped_gemm(*A, *B, offs)

    def frac_row(codes, scales):
        vals = []
        for e in range(k):
            byte = int(codes[e // 2])
            c = (byte >> 4) if e % 2 else (byte & 15)
            q = Fraction(GRID[c & 7]).limit_denominator(2) * (-1 if c & 8 else 1)
            vals.append(q * Fraction(float(E4M3_VALUES[int(scales[e // 16])])))
        return vals

    for g in range(G):
        for r in range(offs[g], offs[g + 1]):
            ar = frac_row(A[0][r], A[1][r])
            for j in range(n):
                br = frac_row(B[0][g][j], B[1][g][j])
                exact = sum(x * y for x, y in zip(ar, br)) * Fraction(float(A[2][r])) * Fraction(float(B[2][g]))
                v = float(exact)
                assert abs(float(out[r, j]) - v) <= abs(v) * 2.0 ** -24 * 1.0001 + 1e-45


def test_gemm_one_hot_rows_give_single_products():
    k, n = 64, 8
    a_codes = np.zeros((k, k // 2), np.uint8)
    for i in range(k):                       # row i has code 7 (6.0) at position i
        a_codes[i, i // 2] = 7 << (4 * (i % 2))
    a_scales = np.full((k, k // 16), 0x38, np.uint8)   # E4M3 1.0
    a_g = np.full(k, 0.5, np.float32)
    rng = np.random.default_rng(23)
    b_codes = rng.integers(0, 256, (1, n, k // 2)).astype(np.uint8)
    b_scales = rng.integers(0x08, 0x7F, (1, n, k // 16)).astype(np.uint8)
    b_g = np.array([0.25], np.float32)
    out = O.grouped_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, np.array([0, k], np.int32))
    b_dq = decode(b_codes[0], b_scales[0], np.full(n, 1.0))
    assert np.array_equal(out, (6.0 * 0.5 * 0.25 * b_dq.T).astype(np.float32))


def test_gemm_at_agrees_and_rows_outside_groups_untouched():
    rng = np.random.default_rng(24)
    rows, G, n, k = 40, 2, 32, 128
    A, B = _random_operands(rng, rows, G, n, k)
    offs = np.array([4, 10, 30], np.int32)
    out = np.full((rows, n), 7.0, np.float32)
    full = O.grouped_gemm(*A, *B, offs)
    assert np.all(full[:4] == 0) and np.all(full[30:] == 0)   # fresh zeros: untouched
    rs = rng.integers(0, rows, 300)
    cs = rng.integers(0, n, 300)
    vals, bnd = O.grouped_gemm_at(*A, *B, offs, rs, cs)
    inside = (rs >= 4) & (rs < 30)
    assert np.array_equal(vals[inside], full[rs[inside], cs[inside]])
    assert np.all(vals[~inside] == 0)
    del out


# ----------------------------------------------------------- SwiGLU/combine --

def test_swiglu_is_nearest_bf16_of_fp64_silu_product():
    rng = np.random.default_rng(25)
    rows, I = 50, 64
    c = (rng.standard_normal((rows, 2 * I)) * 3).astype(np.float32)
    c[0, :I] = 0.0                                    # silu(0) = 0
    prob = rng.random(rows).astype(np.float32)
    prob[1] = 0.0
    d, amax = O.swiglu(c, prob)
    g = torch.from_numpy(c[:, :I].astype(np.float64))
    u = torch.from_numpy(c[:, I:].astype(np.float64))
    v = (torch.nn.functional.silu(g) * u * torch.from_numpy(prob.astype(np.float64))[:, None]).numpy()
    dv = bf16_bits_to_f32(d).astype(np.float64)
    # nearest bf16: the neighbours one step away are not closer
    for step in (-1, 1):
        nb = bf16_bits_to_f32((d.astype(np.int32) + step).astype(np.uint16)).astype(np.float64)
        ok = (np.abs(dv - v) <= np.abs(nb - v) * (1 + 1e-12)) | (v == 0)
        assert ok.all()
    assert np.all(dv[0] == 0) and np.all(dv[1] == 0)
    assert np.array_equal(amax, np.abs(bf16_bits_to_f32(d)).max(axis=1))


def test_combine_matches_numpy_gather_sum():
    rng = np.random.default_rng(26)
    T, k, H, R = 20, 3, 32, 70
    y_rows = rng.standard_normal((R, H)).astype(np.float32)
    dst = rng.integers(-1, R, (T, k)).astype(np.int32)
    y = O.combine(y_rows, dst)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            if dst[t, j] >= 0:
                ref[t] += y_rows[dst[t, j]].astype(np.float64)
    yv = bf16_bits_to_f32(y).astype(np.float64)
    assert np.all(np.abs(yv - ref) <= np.abs(ref) * 2.0 ** -8)


def test_layer_composes_the_steps_and_tracks_the_bf16_layer():
    """Whole-layer oracle: equals the composition of its steps, and stays close
    to the unquantized bf16 layer (loose sanity; the miniTE report measures a
    cosine of about 0.991 for its grouped linear vs BF16)."""
    w = make_moe(0)
    E, I, H = w.experts, w.inter, w.hidden
    w1 = O.quantize(w.w1.reshape(E * 2 * I, H), domain=1,
                    group_offsets=np.arange(E + 1, dtype=np.int32) * 2 * I)
    w2 = O.quantize(w.w2.reshape(E * H, I), domain=1,
                    group_offsets=np.arange(E + 1, dtype=np.int32) * H)
    W1 = (w1[0].reshape(E, 2 * I, H // 2), w1[1].reshape(E, 2 * I, H // 16), w1[2])
    W2 = (w2[0].reshape(E, H, I // 2), w2[1].reshape(E, H, I // 16), w2[2])
    y, b = O.moe_forward(w.x, w.topk_idx, w.topk_prob, E, I, W1, W2)
    rows = b["offsets"][-1]
    c = O.grouped_gemm(b["a1_codes"], b["a1_scales"], b["a1_gscale"], *W1, b["offsets"])
    assert np.array_equal(c[:rows], b["c_fc1"][:rows])
    d, am = O.swiglu(c[:rows], b["row_prob"][:rows])
    assert np.array_equal(d, b["d"][:rows]) and np.array_equal(am, b["amax_d"][:rows])
    a2 = O.quantize(d, amax_in=am)
    assert np.array_equal(a2[0], b["a2_codes"][:rows])
    # bf16 reference layer (fp64 math on the unquantized bf16 operands)
    x = bf16_bits_to_f32(w.x).astype(np.float64)
    W1f = bf16_bits_to_f32(w.w1).astype(np.float64)
    W2f = bf16_bits_to_f32(w.w2).astype(np.float64)
    ref = np.zeros((w.tokens, H))
    for t in range(w.tokens):
        for j in range(w.topk):
            e = w.topk_idx[t, j]
            h = W1f[e] @ x[t]
            act = h[:I] / (1 + np.exp(-h[:I])) * h[I:] * w.topk_prob[t, j]
            ref[t] += W2f[e] @ act
    yq = bf16_bits_to_f32(y).astype(np.float64)
    cos = (yq * ref).sum() / np.linalg.norm(yq) / np.linalg.norm(ref)
    assert cos > 0.95, cos
