"""Pins of the oracle's Four-Over-Six block rule (The 4-bitter Lesson,
"Four-Over-Six for RL Weights and Activations"): a hand-worked row, the
6-candidate against the standard quantizer, the choice against the block
errors of both candidates, and the degenerate rows."""
import json
import os

import numpy as np

from nvfp4_w4a4_quantized_amd.workloads import bf16_bits_to_f32, random_bf16, to_bf16_bits
from oracle import oracle as O

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MSE, MAE = 1, 2


def test_hand_worked_four_over_six_row():
    with open(os.path.join(GOLD, "four_over_six_row.json")) as f:
        g = json.load(f)
    v = np.array(g["x_values"], np.float32)
    x = to_bf16_bits(v)[None]
    assert np.array_equal(bf16_bits_to_f32(x)[0], v)
    for rule, key in ((MSE, "mse"), (MAE, "mae")):
        codes, scales, gs = O.quantize(x, rule=rule)
        assert [f"{b:02x}" for b in scales[0]] == g[key]["expected_scales_hex"], key
        assert [f"{b:02x}" for b in codes[0]] == g[key]["expected_codes_hex"], key
        assert f"{gs.view(np.uint32)[0]:08x}" == g["expected_gscale_hex"]


def _blocks_err(x_f32, deq, metric):
    e = (x_f32.astype(np.float32) - deq.astype(np.float32)).reshape(x_f32.shape[0], -1, 16)
    t = e * e if metric == MSE else np.abs(e)
    acc = np.zeros(t.shape[:2], np.float32)
    for i in range(16):                       # left to right, binary32
        acc = (acc + t[:, :, i]).astype(np.float32)
    return acc


def _deq_f32(codes, scales, gs):
    """q * s_b (exact) times s_g, rounded once to binary32, per element."""
    rows, kh = codes.shape
    q = np.zeros((rows, kh * 2), np.float64)
    q[:, 0::2] = [[O.e2m1_value(int(c) & 15) for c in r] for r in codes]
    q[:, 1::2] = [[O.e2m1_value(int(c) >> 4) for c in r] for r in codes]
    sb = np.repeat(np.array([[O.e4m3_value(int(b)) for b in r] for r in scales]), 16, axis=1)
    return ((q * sb).astype(np.float32) * gs[:, None].astype(np.float32)).astype(np.float32)


def test_six_candidate_is_the_standard_quantizer_at_175_amax_and_choice_minimises_error():
    """With s_g = amax/1536, the 6-candidate of every block is exactly what the
    standard quantizer gives with amax' = 1.75 amax (1.75 amax is exact and
    1.75 amax / 2688 = amax / 1536).  Every block either equals it or, with a
    strictly smaller block error, takes the other candidate, whose codes stay
    within +-4 plus E4M3 rounding."""
    rng = np.random.default_rng(46)
    x = random_bf16(rng, (24, 256), 1.0)
    x[3, :16] = to_bf16_bits(np.full(16, 5.0, np.float32))          # a block that prefers 4
    xf = bf16_bits_to_f32(x)
    amax = np.abs(xf).max(axis=1).astype(np.float32)
    c6, s6, g6 = O.quantize(x, amax_in=(amax * np.float32(1.75)).astype(np.float32))
    for rule in (MSE, MAE):
        c, s, g = O.quantize(x, rule=rule)
        assert np.array_equal(g, g6)
        e6 = _blocks_err(xf, _deq_f32(c6, s6, g6), rule)
        e = _blocks_err(xf, _deq_f32(c, s, g), rule)
        same = (s == s6) & np.all(c.reshape(24, 16, 8) == c6.reshape(24, 16, 8), axis=2)
        assert np.all(e[~same] < e6[~same])
        assert np.all(e[same] == e6[same])
        assert (~same).sum() > 0 and same.sum() > 0
        # the other candidate maps the block maximum to about 4: no code above 4.0 (index 6)
        nib = np.stack([c & 15, c >> 4], axis=-1).reshape(24, 16, 16) & 7
        assert nib[~same].max() <= 6


def test_four_over_six_zero_and_sign_rows():
    x = np.zeros((2, 32), np.uint16)
    x[1, 5] = 0x8000                                   # -0.0
    for rule in (MSE, MAE):
        c, s, g = O.quantize(x, rule=rule)
        assert np.all(g == 0) and np.all(s == 0)
        assert c[0].sum() == 0 and c[1, 2] == 0x80     # element 5: high nibble of byte 2


def test_group_domain_uses_the_four_over_six_outer_scale():
    rng = np.random.default_rng(47)
    x = random_bf16(rng, (6, 64), 0.3)
    offs = np.array([0, 2, 6], np.int32)
    c, s, g = O.quantize(x, domain=1, group_offsets=offs, rule=MSE)
    xf = bf16_bits_to_f32(x)
    for gi in range(2):
        amax = np.float32(np.abs(xf[offs[gi]:offs[gi + 1]]).max())
        assert g[gi] == np.float32(amax / np.float32(1536.0))
        rc, rs, rg = O.quantize(x[offs[gi]:offs[gi + 1]],
                                amax_in=np.full(offs[gi + 1] - offs[gi], amax, np.float32),
                                rule=MSE)
        assert np.array_equal(c[offs[gi]:offs[gi + 1]], rc)
        assert np.array_equal(s[offs[gi]:offs[gi + 1]], rs)
