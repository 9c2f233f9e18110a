"""Pins of the oracle's outer-scale domains beyond per-token: the per-tensor
scale (one group covering every row) and 16x16 two-dimensional weight blocks
(miniTE Technical Report §2.2 "two-dimensional block-scaled quantization",
App. D2 "2D weight quantization")."""
import numpy as np
import pytest

from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, random_bf16
from oracle import oracle as O


def _q2d(x, offs):
    return O.quantize(x, domain=2, group_offsets=np.asarray(offs, np.int32))


def test_2d_blocks_of_identical_rows_equal_1d():
    """A tile whose 16 rows are equal has the 1D block maximum as its tile
    maximum: domain 2 reduces to domain 1."""
    rng = np.random.default_rng(61)
    base = random_bf16(rng, (6, 96), 0.5)
    x = np.repeat(base, 16, axis=0)                     # 6 tiles of identical rows
    offs = [0, 32, 96]
    c2, s2, g2 = _q2d(x, offs)
    c1, s1, g1 = O.quantize(x, domain=1, group_offsets=np.asarray(offs, np.int32))
    assert np.array_equal(g2, g1) and np.array_equal(s2, s1) and np.array_equal(c2, c1)


def _codes_grid(c):
    rows = c.shape[0]
    out = np.zeros((rows, c.shape[1] * 2), np.uint8)
    out[:, 0::2] = c & 15
    out[:, 1::2] = c >> 4
    return out


def test_2d_quantization_is_transpose_consistent():
    """Every element's code depends only on its 16x16 tile and the outer scale,
    so quantizing W and W^T gives transposed codes and scales."""
    rng = np.random.default_rng(62)
    w = random_bf16(rng, (64, 96), 0.02)
    c, s, g = _q2d(w, [0, 64])
    ct, st, gt = _q2d(np.ascontiguousarray(w.T), [0, 96])
    assert g[0] == gt[0]
    assert np.array_equal(_codes_grid(c), _codes_grid(ct).T)
    tiles = s[::16]                                      # [64/16, 96/16]
    tiles_t = st[::16]                                   # [96/16, 64/16]
    assert np.array_equal(tiles, tiles_t.T)
    for r in range(64):                                  # the scale repeats in a tile's rows
        assert np.array_equal(s[r], tiles[r // 16])


def test_2d_tile_scale_is_the_1d_scale_of_the_row_holding_the_tile_maximum():
    rng = np.random.default_rng(63)
    w = random_bf16(rng, (32, 64), 0.1)
    wf = bf16_bits_to_f32(w)
    c2, s2, g2 = _q2d(w, [0, 32])
    c1, s1, g1 = O.quantize(w, domain=1, group_offsets=np.array([0, 32], np.int32))
    assert g1[0] == g2[0]
    for t in range(2):
        for b in range(4):
            tile = np.abs(wf[16 * t:16 * t + 16, 16 * b:16 * b + 16])
            rmax = 16 * t + int(np.argmax(tile.max(axis=1)))
            assert np.all(s2[16 * t:16 * t + 16, b] == s1[rmax, b])
            assert np.array_equal(c2[rmax, 8 * b:8 * b + 8], c1[rmax, 8 * b:8 * b + 8])


def test_2d_rejects_ragged_groups_and_other_rules():
    x = np.zeros((48, 32), np.uint16)
    with pytest.raises(ValueError):
        _q2d(x, [0, 8, 48])
    with pytest.raises(ValueError):
        O.quantize(x, domain=2, group_offsets=np.array([0, 48], np.int32), rule=1)


def test_per_tensor_scale_depends_on_the_batch_but_per_token_does_not():
    """miniTE Technical Report §2.3 (per-tensor against per-token outer
    scales).  One token is quantized in two batches with different
    neighbours.  Under one outer scale for the whole tensor, its codes and
    scale change with the neighbours.  Under its own per-token scale, both
    batches give it the same bits."""
    rng = np.random.default_rng(64)
    tok = random_bf16(rng, (1, 128), 1.0)
    ctx_a = random_bf16(rng, (3, 128), 1.0)
    ctx_b = random_bf16(rng, (3, 128), 40.0)
    xa, xb = np.concatenate([tok, ctx_a]), np.concatenate([tok, ctx_b])
    one = lambda n: np.array([0, n], np.int32)
    ta = O.quantize(xa, domain=1, group_offsets=one(4))
    tb = O.quantize(xb, domain=1, group_offsets=one(4))
    assert ta[2][0] != tb[2][0] and not np.array_equal(ta[0][0], tb[0][0])
    pa, pb = O.quantize(xa), O.quantize(xb)
    assert np.array_equal(pa[0][0], pb[0][0]) and pa[2][0] == pb[2][0]
