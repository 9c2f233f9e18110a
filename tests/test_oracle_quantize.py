"""Pins of the oracle's NVFP4 quantizer: the hand-worked row, exact lattice
idempotence, power-of-two equivariance, sign symmetry, per-row independence
(the context-swap property of the miniTE summary, App. D), zero rows,
extreme inputs, the reconstruction error bound and the group (per-expert)
domain.  Decoding in these tests uses the printed grid and torch's E4M3
decode, not the oracle's decode."""
import json
import os

import numpy as np
import torch

from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, to_bf16_bits
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLD, "e2m1_grid.json")) as _f:
    GRID = np.array(json.load(_f)["magnitudes"], np.float64)
E4M3_VALUES = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def decode(codes, scales, gscale_rows):
    """Independent decode: x^ = q * s_b * s_g with the printed grid."""
    codes = np.asarray(codes)
    lo = codes & 15
    hi = codes >> 4
    nib = np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)
    q = GRID[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    sb = np.repeat(E4M3_VALUES[np.asarray(scales)], 16, axis=1)
    return q * sb * np.asarray(gscale_rows, np.float64)[:, None]


def test_hand_worked_row():
    with open(os.path.join(GOLD, "worked_row.json")) as f:
        g = json.load(f)
    x = np.array([[int(h, 16) for h in g["x_bf16_hex"]]], np.uint16)
    assert np.array_equal(bf16_bits_to_f32(x)[0], np.array(g["x_values"], np.float32))
    codes, scales, gs = O.quantize(x)
    assert [f"{b:02x}" for b in codes[0]] == g["expected_codes_hex"]
    assert [f"{b:02x}" for b in scales[0]] == g["expected_scales_hex"]
    assert f"{gs.view(np.uint32)[0]:08x}" == g["expected_gscale_hex"]


def test_hand_worked_tie_row():
    """Exact quotient ties with an inexact reciprocal: the decision uses the
    correctly rounded binary32 quotient."""
    with open(os.path.join(GOLD, "tie_row.json")) as f:
        g = json.load(f)
    v = np.array(g["x_values"], np.float32)
    x = to_bf16_bits(v)[None]
    assert np.array_equal(bf16_bits_to_f32(x)[0], v)
    codes, scales, gs = O.quantize(x)
    assert [f"{b:02x}" for b in codes[0]] == g["expected_codes_hex"]
    assert [f"{b:02x}" for b in scales[0]] == g["expected_scales_hex"]
    assert f"{gs.view(np.uint32)[0]:08x}" == g["expected_gscale_hex"]


def _lattice_rows(rng, rows, k, j):
    """x = q * s_b * 2^j with >= one +-6 code per block and one block at 448."""
    nb = k // 16
    normal_bytes = np.arange(0x08, 0x7F)           # normal E4M3 scales
    codes = rng.integers(0, 16, size=(rows, k)).astype(np.uint8)
    for r in range(rows):
        for b in range(nb):
            pos = rng.integers(0, 16)
            codes[r, b * 16 + pos] = 7 | (8 if rng.random() < 0.5 else 0)
    sb = rng.choice(normal_bytes, size=(rows, nb)).astype(np.uint8)
    sb[np.arange(rows), rng.integers(0, nb, size=rows)] = 0x7E
    q = GRID[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    x = q * np.repeat(E4M3_VALUES[sb], 16, axis=1) * 2.0 ** j
    xb = to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(xb).astype(np.float64), x)   # exact in bf16
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    # zero magnitudes may carry either sign in x; the encoder keeps x's sign
    return xb, packed, sb


def test_lattice_points_quantize_to_themselves():
    rng = np.random.default_rng(10)
    for j in (-12, -8, -3, 0, 2, 7):
        xb, packed, sb = _lattice_rows(rng, 16, 256, j)
        codes, scales, gs = O.quantize(xb)
        assert np.array_equal(scales, sb)
        assert np.all(gs == np.float32(2.0 ** j))
        # compare magnitudes exactly; signs of zero follow x (which is +-0 per q sign)
        assert np.array_equal(codes & 0x77, packed & 0x77)
        xs = bf16_bits_to_f32(xb)
        sign_x = np.signbit(xs).astype(np.uint8)
        sign_c = np.stack([(codes >> 3) & 1, (codes >> 7) & 1], -1).reshape(xs.shape)
        assert np.array_equal(sign_x, sign_c)


def test_power_of_two_equivariance():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    xb = to_bf16_bits(x)
    c0, s0, g0 = O.quantize(xb)
    for j in (-30, -9, -1, 1, 5, 20):
        xj = to_bf16_bits(bf16_bits_to_f32(xb) * np.float32(2.0 ** j))
        c1, s1, g1 = O.quantize(xj)
        assert np.array_equal(c1, c0)
        assert np.array_equal(s1, s0)
        assert np.array_equal(g1, g0 * np.float32(2.0 ** j))


def test_sign_symmetry():
    rng = np.random.default_rng(12)
    xb = to_bf16_bits(rng.standard_normal((16, 256)).astype(np.float32))
    c0, s0, g0 = O.quantize(xb)
    c1, s1, g1 = O.quantize(xb ^ np.uint16(0x8000))
    assert np.array_equal(c1, c0 ^ np.uint8(0x88))
    assert np.array_equal(s1, s0)
    assert np.array_equal(g1, g0)


def test_rows_are_independent_context_swap():
    """A target row's payload does not depend on the other rows (per-token
    outer scale; miniTE summary App. D context-swap checks)."""
    rng = np.random.default_rng(13)
    base = to_bf16_bits(rng.standard_normal((8, 256)).astype(np.float32))
    c0, s0, g0 = O.quantize(base)
    for _ in range(6):
        other = to_bf16_bits((rng.standard_normal((8, 256)) * rng.uniform(0.01, 1000)).astype(np.float32))
        other[3] = base[3]
        c1, s1, g1 = O.quantize(other)
        assert np.array_equal(c1[3], c0[3]) and np.array_equal(s1[3], s0[3]) and g1[3] == g0[3]


def test_zero_rows():
    x = np.zeros((2, 64), np.uint16)
    x[1] = 0x8000  # -0.0
    c, s, g = O.quantize(x)
    assert np.all(s == 0) and np.all(g == 0)
    assert np.all(c[0] == 0) and np.all(c[1] == 0x88)


def test_extreme_inputs_saturate_or_underflow_without_nan():
    rows = []
    big = np.float32(3.3895314e38)      # largest finite bf16
    rows.append(np.full(64, big, np.float32))
    rows.append(np.linspace(-float(big), float(big), 64).astype(np.float32))
    rows.append(np.full(64, 1e-40, np.float32))           # bf16 subnormals
    tiny = np.zeros(64, np.float32); tiny[5] = 9.2e-41
    rows.append(tiny)
    mix = np.ones(64, np.float32) * 1e-30; mix[0] = 1e30
    rows.append(mix)
    xb = to_bf16_bits(np.stack(rows))
    c, s, g = O.quantize(xb)
    assert np.all(np.isfinite(g))
    assert not np.any((s & 0x7F) == 0x7F)
    dq = decode(c, s, g)
    assert np.all(np.isfinite(dq))


def test_reconstruction_error_within_one_decode_step():
    """|x - x^| <= d_b = s_b*s_g for every element of a block with a normal
    E4M3 scale (rounding error <= 1 grid step of 2 * d/2; clipping <= 0.5 d)."""
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-5, 5, (64, 1)))).astype(np.float32)
    xb = to_bf16_bits(x)
    c, s, g = O.quantize(xb)
    dq = decode(c, s, g)
    d = np.repeat(E4M3_VALUES[s], 16, axis=1) * g[:, None].astype(np.float64)
    normal = np.repeat(s >= 0x08, 16, axis=1)
    err = np.abs(dq - bf16_bits_to_f32(xb).astype(np.float64))
    # slack 2^-20: the quotient x/d is rounded to binary32 before the grid
    # decision, so a value a hair above a midpoint can land on it
    assert np.all(err[normal] <= d[normal] * (1 + 2.0 ** -20))
    snr = 20 * np.log10(np.linalg.norm(bf16_bits_to_f32(xb)) / np.linalg.norm(dq - bf16_bits_to_f32(xb)))
    assert 15.0 < snr < 25.0   # sanity: the miniTE report quotes ~19.9 dB for E2M1 + E4M3 scales


def test_amax_in_is_the_outer_scale_domain():
    """Quantizing x with amax_in = A equals quantizing x next to a block whose
    maximum is A (the amax reuse of miniTE §5.3 skips only the reduction)."""
    rng = np.random.default_rng(15)
    x = rng.standard_normal((4, 128)).astype(np.float32)
    xb = to_bf16_bits(x)
    amax = np.abs(bf16_bits_to_f32(xb)).max(axis=1)
    A = (amax * np.float32(3.0)).astype(np.float32)
    A = bf16_bits_to_f32(to_bf16_bits(A))
    ext = np.concatenate([xb, to_bf16_bits(np.repeat(A[:, None], 16, axis=1))], axis=1)
    c_ext, s_ext, g_ext = O.quantize(ext)
    c_in, s_in, g_in = O.quantize(xb, amax_in=A)
    assert np.array_equal(c_in, c_ext[:, :64])
    assert np.array_equal(s_in, s_ext[:, :8])
    assert np.array_equal(g_in, g_ext)
    c0, s0, g0 = O.quantize(xb)
    c1, s1, g1 = O.quantize(xb, amax_in=np.abs(bf16_bits_to_f32(xb)).max(axis=1))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1) and np.array_equal(g0, g1)


def test_group_domain_is_row_domain_with_the_group_amax():
    rng = np.random.default_rng(16)
    x = to_bf16_bits((rng.standard_normal((24, 128)) * rng.uniform(0.1, 10, (24, 1))).astype(np.float32))
    offs = np.array([0, 5, 5, 17, 24], np.int32)         # includes an empty group
    c, s, g = O.quantize(x, domain=1, group_offsets=offs)
    xf = np.abs(bf16_bits_to_f32(x))
    for gi in range(4):
        r0, r1 = offs[gi], offs[gi + 1]
        if r1 == r0:
            assert g[gi] == 0
            continue
        A = xf[r0:r1].max()
        assert g[gi] == np.float32(A) / np.float32(2688.0)
        cr, sr, gr = O.quantize(x[r0:r1], amax_in=np.full(r1 - r0, A, np.float32))
        assert np.array_equal(c[r0:r1], cr) and np.array_equal(s[r0:r1], sr)
    # changing a row of another group leaves group 3 unchanged
    x2 = x.copy(); x2[0] = to_bf16_bits(np.full(128, 1e4, np.float32))
    c2, s2, g2 = O.quantize(x2, domain=1, group_offsets=offs)
    assert np.array_equal(c2[17:], c[17:]) and g2[3] == g[3]
