"""Pins of the oracle's single-pass path (O12; miniTE Technical Report §5.6,
"Exploring Single-Pass Fusion"): FC2 consumes the activation in K-tiles,
each quantized with the outer scale of the row's running amax, and the FC2
partial sums are converted to the new scale whenever it grows.

What fixes it independently of the oracle code:
  - a hand-worked three-tile row (tests/golden/single_pass_row.json);
  - reductions to the two-pass path, which the other pins fix: one tile
    spanning the row, and rows whose maximum lies in their first tile;
  - invariants: the tile scales are the running maximum (non-decreasing, the
    last equals the two-pass scale), and a row whose maximum lies in its last
    tile ends with the two-pass codes there;
  - the FC2 equals numpy's float64 matmul of the fully dequantized operands
    (each activation element scaled by the gs of its own tile), decoded here
    with the printed grid and torch's E4M3 decode;
  - zero rows give zero."""
import json
import os

import numpy as np
import pytest
import torch

from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, random_bf16, to_bf16_bits
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
with open(os.path.join(GOLD, "e2m1_grid.json")) as _f:
    GRID = np.array(json.load(_f)["magnitudes"], np.float64)
E4M3_VALUES = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _qsb(codes, scales):
    """q * s_b per element (outer scales excluded), printed grid + torch E4M3."""
    codes = np.asarray(codes)
    nib = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    q = GRID[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    return q * np.repeat(E4M3_VALUES[np.asarray(scales)], 16, axis=1)


def _weights(rng, G, n, k):
    from gpu_util import oracle_weights
    return oracle_weights(random_bf16(rng, (G, n, k), 0.02))


def test_hand_worked_three_tile_row():
    with open(os.path.join(GOLD, "single_pass_row.json")) as f:
        g = json.load(f)
    x = np.array([[int(h, 16) for h in r] for r in g["x_bf16_hex"]], np.uint16)
    assert np.array_equal(bf16_bits_to_f32(x), np.array(g["x_values"], np.float32))
    tile = g["tile"]
    codes, scales, gs = O.online_quantize(x, tile)
    for r in range(2):
        assert [f"{b:02x}" for b in codes[r]] == g["expected_codes_hex"][r]
        assert [f"{b:02x}" for b in scales[r]] == g["expected_scales_hex"][r]
        assert [f"{v:08x}" for v in gs[r].view(np.uint32)] == g["expected_gs_hex"][r]
    wr = g["weight_row"]
    k = x.shape[1]
    W = (np.full((1, 1, k // 2), int(wr["codes_byte"], 16), np.uint8),
         np.full((1, 1, k // 16), int(wr["scale_byte"], 16), np.uint8),
         np.array([wr["gscale"]], np.float32))
    y = O.single_pass_gemm(codes, scales, gs, tile, *W, np.array([0, 2], np.int32))
    assert y[:, 0].tolist() == g["expected_y"]
    assert y[0, 0] != g["expected_y_without_rescale"]


def test_one_tile_spanning_the_row_is_the_two_pass_path():
    rng = np.random.default_rng(3)
    p = random_bf16(rng, (40, 96), 0.3)
    p[5] = 0
    c1, s1, g1 = O.online_quantize(p, 96)
    c2, s2, g2 = O.quantize(p)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(g1[:, 0].view(np.uint32), g2.view(np.uint32))
    # a tile wider than the row is the same single tile
    c3, s3, g3 = O.online_quantize(p, 1024)
    assert np.array_equal(c3, c1) and np.array_equal(g3, g1)
    # and its FC2 is the grouped GEMM bit for bit (same sums, same order)
    W = _weights(rng, 2, 64, 96)
    offs = np.array([0, 17, 40], np.int32)
    y1 = O.single_pass_gemm(c1, s1, g1, 96, *W, offs)
    y2 = O.grouped_gemm(c2, s2, g2, *W, offs)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_row_maximum_in_the_first_tile_gives_the_two_pass_codes():
    rng = np.random.default_rng(4)
    p = random_bf16(rng, (64, 768), 0.5)
    pv = bf16_bits_to_f32(p)
    # put each row's maximum magnitude into its first tile
    big = np.abs(pv).max(axis=1) * 1.5
    p[:, 3] = to_bf16_bits(np.where(rng.random(64) < 0.5, -big, big).astype(np.float32))
    c1, s1, g1 = O.online_quantize(p, 256)
    c2, s2, g2 = O.quantize(p)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.all(g1.view(np.uint32) == g2.view(np.uint32)[:, None])
    W = _weights(rng, 1, 32, 768)
    offs = np.array([0, 64], np.int32)
    y1, b1 = O.single_pass_gemm(c1, s1, g1, 256, *W, offs, with_bound=True)
    y2 = O.grouped_gemm(c2, s2, g2, *W, offs)
    # the same exact products summed tile by tile (fp64): equal up to fp64
    # rounding before the final binary32 rounding
    assert np.all(np.abs(y1.astype(np.float64) - y2) <= 2.0 ** -40 * b1 + np.abs(y2) * 2.0 ** -23)


def test_tile_scales_are_the_running_maximum():
    rng = np.random.default_rng(5)
    p = random_bf16(rng, (200, 768), 1.0)
    pv = bf16_bits_to_f32(p)
    # rows whose tiles grow, shrink or jump
    p[:50] = to_bf16_bits(pv[:50] * np.repeat(np.array([0.25, 1.0, 4.0], np.float32), 256))
    p[50:100] = to_bf16_bits(pv[50:100] * np.repeat(np.array([4.0, 1.0, 0.25], np.float32), 256))
    p[100:110] = 0
    c, s, gs = O.online_quantize(p, 256)
    assert np.all(np.diff(gs, axis=1) >= 0)
    _, _, g2 = O.quantize(p)
    assert np.array_equal(gs[:, -1].view(np.uint32), g2.view(np.uint32))
    # growing rows change scale at every tile; shrinking rows never do
    assert np.all(gs[:50, 0] < gs[:50, 1]) and np.all(gs[:50, 1] < gs[:50, 2])
    assert np.all(gs[50:100, 0] == gs[50:100, 2])
    # rows whose maximum lies in the last tile end with the two-pass codes there
    c2, s2, _ = O.quantize(p)
    last = slice(512 // 2, 768 // 2)
    assert np.array_equal(c[:50, last], c2[:50, last])
    assert np.array_equal(s[:50, 32:], s2[:50, 32:])
    # ... while their earlier tiles were quantized with smaller scales
    assert not np.array_equal(s[:50, :16], s2[:50, :16])


@pytest.mark.parametrize("tile", [16, 128, 256, 320])
def test_fc2_is_the_dequantized_product(tile):
    """Y = sum_i gs_i * gs_W * dO_i, i.e. the product of the fully dequantized
    operands, whatever the order of the rescales."""
    rng = np.random.default_rng(tile)
    k, n, G = 768, 48, 3
    p = random_bf16(rng, (90, k), 1.0)
    pv = bf16_bits_to_f32(p)
    p[:30] = to_bf16_bits(pv[:30] * np.linspace(0.1, 3.0, k, dtype=np.float32))
    p[40] = 0
    codes, scales, gs = O.online_quantize(p, tile)
    W = _weights(rng, G, n, k)
    offs = np.array([0, 25, 25, 90], np.int32)
    y, bound = O.single_pass_gemm(codes, scales, gs, tile, *W, offs, with_bound=True)
    nt = O.num_tiles(k, tile)
    col_tile = np.minimum(np.arange(k) // tile, nt - 1)
    a = _qsb(codes, scales) * gs[:, col_tile].astype(np.float64)
    for g in range(G):
        r0, r1 = offs[g], offs[g + 1]
        if r0 == r1:
            continue
        b = _qsb(W[0][g], W[1][g]) * np.float64(W[2][g])
        ref = a[r0:r1] @ b.T
        babs = np.abs(a[r0:r1]) @ np.abs(b).T
        assert np.all(np.abs(y[r0:r1] - ref) <= np.abs(ref) * 2.0 ** -23 + babs * 2.0 ** -40)
        assert np.allclose(bound[r0:r1], babs, rtol=1e-12, atol=0)
    assert np.all(y[40] == 0)


def test_zero_rows_give_zero():
    p = np.zeros((3, 64), np.uint16)
    p[1, 7] = 0x8000                       # -0.0
    codes, scales, gs = O.online_quantize(p, 32)
    assert np.all(gs == 0) and np.all(scales == 0)
    assert codes[1, 3] == 0x80 and np.count_nonzero(codes) == 1
    rng = np.random.default_rng(9)
    W = _weights(rng, 1, 32, 64)
    y = O.single_pass_gemm(codes, scales, gs, 32, *W, np.array([0, 3], np.int32))
    assert np.all(y == 0) and not np.any(np.signbit(y) & (y != 0))


def test_layer_with_one_tile_equals_the_two_pass_layer():
    from gpu_util import moe_case
    w, W1, W2 = moe_case(0)
    y1, b1 = O.moe_forward_single_pass(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2,
                                       tile=w.inter)
    y2, b2 = O.moe_forward(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2)
    assert np.array_equal(y1, y2)
    # with four tiles the layer moves only by the quantization differences
    y4, b4 = O.moe_forward_single_pass(w.x, w.topk_idx, w.topk_prob, w.experts, w.inter, W1, W2,
                                       tile=32)
    a = bf16_bits_to_f32(y4).astype(np.float64)
    b = bf16_bits_to_f32(y2).astype(np.float64)
    assert 0 < np.linalg.norm(a - b) / np.linalg.norm(b) < 5e-2
    assert np.array_equal(b4["d"], b2["d"])          # FC1 and SwiGLU are unchanged
