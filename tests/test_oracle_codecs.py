"""Pins of the oracle's element/scale codecs against what the pages print and
against library routines (torch's float8_e4m3fn and bfloat16 casts)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _grid():
    with open(os.path.join(GOLD, "e2m1_grid.json")) as f:
        return json.load(f)


def test_e2m1_decode_matches_printed_grid():
    g = _grid()["magnitudes"]
    for code in range(16):
        v = O.e2m1_value(code)
        mag = g[code & 7]
        assert abs(v) == mag
        assert (np.signbit(v)) == bool(code & 8)


def test_e2m1_encode_is_identity_on_grid():
    g = _grid()["magnitudes"]
    for i, m in enumerate(g):
        assert O.e2m1_encode(m) == i
        assert O.e2m1_encode(-m) == (i | 8)


def _f32_neighbourhood(vals, ulps=3):
    out = []
    for v in vals:
        b = np.array([v], np.float32).view(np.uint32)[0]
        for d in range(-ulps, ulps + 1):
            if int(b) + d < 0:
                continue
            bb = np.uint32(int(b) + d)
            out.append(np.array([bb], np.uint32).view(np.float32)[0])
    return np.array(out, np.float32)


def test_e2m1_encode_is_round_to_nearest_even_on_grid():
    """Brute force: the chosen magnitude is a nearest grid value, and exact
    midpoints go to the even index (round-to-nearest-even)."""
    g = np.array(_grid()["magnitudes"], np.float64)
    mids = (g[1:] + g[:-1]) / 2
    rng = np.random.default_rng(0)
    samples = np.concatenate([
        _f32_neighbourhood(np.concatenate([g, mids]), 4),
        rng.uniform(0, 7, 20000).astype(np.float32),
        np.array([0.0, 1e-30, 5.9999995, 6.0, 6.0000005, 1e30, np.inf], np.float32)])
    samples = samples[samples >= 0]
    for r in samples:
        code = O.e2m1_encode(float(r))
        assert code < 8
        if r >= 6:
            assert code == 7
            continue
        dist = np.abs(g - np.float64(r))
        best = dist.min()
        assert dist[code] == best, (r, code)
        tied = np.flatnonzero(dist == best)
        if tied.size == 2:
            assert code % 2 == 0, (r, code)


def test_e2m1_encode_sign_of_zero_and_negatives():
    assert O.e2m1_encode(-0.0) == 8
    assert O.e2m1_encode(0.0) == 0
    assert O.e2m1_encode(-0.1) == 8          # rounds to zero, keeps its sign
    assert O.e2m1_encode(-5.0) == 8 | 6      # tie 4/6 -> even index (4)
    assert O.e2m1_encode(-1e9) == 15


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    allb = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = O.e4m3_value(b)
        if np.isnan(allb[b]):
            assert np.isnan(v), b
        else:
            assert v == allb[b], (b, v, allb[b])
    assert O.e4m3_value(0x7E) == _grid()["e4m3_max_implied"]  # 448 = 2688 / 6


def test_e4m3_encode_matches_torch_cast_below_448():
    grid = np.array([O.e4m3_value(b) for b in range(0x7F)], np.float64)
    mids = (grid[1:] + grid[:-1]) / 2
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        _f32_neighbourhood(np.concatenate([grid, mids]), 3),
        rng.uniform(0, 448, 200000).astype(np.float32),
        np.exp(rng.uniform(np.log(1e-6), np.log(448), 200000)).astype(np.float32)])
    vals = vals[(vals >= 0) & (vals <= 448)]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([O.e4m3_encode(float(v)) for v in vals], np.uint8)
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, (vals[bad[:5]], ours[bad[:5]], ref[bad[:5]])


def test_e4m3_encode_saturates_above_448():
    for v in [448.0, 448.5, 463.9, 464.0, 470.0, 1e6, 3.4e38]:
        assert O.e4m3_encode(v) == 0x7E


def test_f64_to_bf16_matches_torch_for_binary32_values():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(50000).astype(np.float32) * 10,
                        _f32_neighbourhood(np.array([1.0, 1.00390625, 1.005859375, 3.0], np.float32), 40)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.uint16).numpy()
    ours = np.array([O.f64_to_bf16(float(x)) for x in v], np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_is_nearest_for_fp64_values():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))
    for x in v:
        h = O.f64_to_bf16(float(x))
        hv = float(np.array([h << 16], np.uint32).view(np.float32)[0])
        # neighbours one bf16 step either side are not closer
        for dh in (-1, 1):
            nv = float(np.array([(h + dh) << 16], np.uint32).view(np.float32)[0])
            assert abs(hv - x) <= abs(nv - x)
