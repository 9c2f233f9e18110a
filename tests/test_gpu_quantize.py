"""GPU parity of nvfp4_quantize (through the C ABI) against the oracle:
codes, E4M3 block scales and FP32 outer scales must match bit for bit."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, moe_case, oracle_weights, say
from nvfp4_w4a4_quantized_amd.workloads import make_dense, to_bf16_bits
from oracle import oracle as O

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _ops():
    from nvfp4_w4a4_quantized_amd import ops
    return ops


def _check_rows(xb: np.ndarray, what: str, amax_in=None):
    say("nvfp4_quantize", what, xb.shape)
    c, s, g = _ops().nvfp4_quantize(dev_bf16(xb), amax_in=None if amax_in is None else dev(amax_in))
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(xb, amax_in=amax_in)
    assert np.array_equal(host(s), rs), f"{what}: scales differ"
    assert np.array_equal(host(g).view(np.uint32), rg.view(np.uint32)), f"{what}: outer scales differ"
    hc = host(c)
    if not np.array_equal(hc, rc):
        bad = np.argwhere(hc != rc)
        r, b = bad[0]
        raise AssertionError(f"{what}: {len(bad)} code bytes differ; first row {r} byte {b}: "
                             f"gpu {hc[r, b]:02x} oracle {rc[r, b]:02x}")


def test_golden_rows():
    for name in ("worked_row.json", "tie_row.json"):
        with open(os.path.join(GOLD, name)) as f:
            gold = json.load(f)
        xb = to_bf16_bits(np.array(gold["x_values"], np.float32))[None]
        c, s, g = _ops().nvfp4_quantize(dev_bf16(xb))
        torch.cuda.synchronize()
        assert [f"{b:02x}" for b in host(c)[0]] == gold["expected_codes_hex"], name
        assert [f"{b:02x}" for b in host(s)[0]] == gold["expected_scales_hex"], name
        assert f"{host(g).view(np.uint32)[0]:08x}" == gold["expected_gscale_hex"], name


@pytest.mark.parametrize("wid", [0, 2, 3, 4])
def test_moe_activations(wid):
    w, _, _ = moe_case(wid, with_weights=False)
    _check_rows(w.x, f"moe workload {wid} activations")


def test_dense_projection_inputs():
    d = make_dense()
    for pname, x, _ in d.projections:
        _check_rows(x, f"dense {pname} input")


@pytest.mark.parametrize("k", [16, 32, 48, 144, 768, 1040, 2048, 4096, 16384])
def test_shapes_and_distributions(k):
    rng = np.random.default_rng(100 + k)
    rows = 67
    x = (rng.standard_normal((rows, k)) * np.exp(rng.uniform(-30, 30, (rows, 1)))).astype(np.float32)
    x[3] = 0.0
    x[4] = -0.0
    x[5, ::7] = 1e-38
    x[6] = rng.standard_t(3, size=k) * 100
    x[7, : min(k, 16)] = 3.3895314e38
    _check_rows(to_bf16_bits(x), f"random k={k}")


def test_lattice_ties_and_extremes():
    """Exact grid points and quotient ties exercise the exact-division path."""
    rng = np.random.default_rng(7)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5])
    rows = []
    for j in (-120, -60, -8, 0, 9, 100):
        for sb in (0x01, 0x07, 0x08, 0x0F, 0x33, 0x63, 0x7E):
            sv = float(torch.tensor([sb], dtype=torch.uint8).view(torch.float8_e4m3fn).float())
            q = rng.choice(grid, size=256) * rng.choice([-1, 1], size=256)
            q[0] = 6.0
            row = q * sv * 2.0 ** j
            row[16] = 6 * 448 * 2.0 ** j          # fixes amax: s_g = 2^j
            rows.append(row)
    x = np.array(rows)
    x = np.where(np.isfinite(x) & (np.abs(x) < 3e38), x, 0.0).astype(np.float32)
    _check_rows(to_bf16_bits(x), "lattice and ties")


def test_amax_in_and_leading_dimension():
    rng = np.random.default_rng(8)
    xb = to_bf16_bits(rng.standard_normal((40, 256)).astype(np.float32))
    am = (np.abs(rng.standard_normal(40)) * 5).astype(np.float32)
    am[0] = 0.0
    _check_rows(xb, "amax_in", amax_in=am)
    # ld_x > k through the C ABI directly
    from nvfp4_w4a4_quantized_amd import _lib
    big = to_bf16_bits(rng.standard_normal((40, 384)).astype(np.float32))
    xd = dev_bf16(big)
    c = torch.empty((40, 128), dtype=torch.uint8, device="cuda")
    s = torch.empty((40, 16), dtype=torch.uint8, device="cuda")
    g = torch.empty(40, dtype=torch.float32, device="cuda")
    say("nvfp4_quantize ld_x=384 k=256")
    _lib.check(_lib.lib().nvfp4_quantize(_lib.ptr(xd), 40, 256, 384, 0, None, 0, None, 0,
                                         _lib.ptr(c), _lib.ptr(s), _lib.ptr(g),
                                         _lib.stream_handle()), "quantize ld")
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(np.ascontiguousarray(big[:, :256]))
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs) and np.array_equal(host(g), rg)


def test_group_domain_with_empty_groups():
    rng = np.random.default_rng(9)
    xb = to_bf16_bits((rng.standard_normal((50, 512)) * rng.uniform(0.01, 100, (50, 1))).astype(np.float32))
    offs = np.array([0, 7, 7, 30, 30, 50], np.int32)
    say("nvfp4_quantize groups")
    c, s, g = _ops().nvfp4_quantize(dev_bf16(xb), scale_domain=1, group_offsets=dev(offs))
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(xb, domain=1, group_offsets=offs)
    assert np.array_equal(host(c), rc) and np.array_equal(host(s), rs)
    assert np.array_equal(host(g), rg)


@pytest.mark.parametrize("k", [256, 2048])
def test_group_domain_across_waves(k):
    """Groups spanning several 64-row waves of the group-amax reduction and
    boundaries inside the encoder's waves, with each group's maximum planted
    in a different wave (the per-wave partial maxima must combine)."""
    rng = np.random.default_rng(k)
    rows = 700
    x = (rng.standard_normal((rows, k)) * 0.5).astype(np.float32)
    offs = np.array([0, 100, 100, 333, 334, 700], np.int32)
    for g, r in enumerate([90, 0, 150, 333, 650]):
        if offs[g] <= r < offs[g + 1]:
            x[r, (7 * g) % k] = 40.0 + g          # the group's maximum
    xb = to_bf16_bits(x)
    say("nvfp4_quantize groups across waves", k)
    c, s, gsc = _ops().nvfp4_quantize(dev_bf16(xb), scale_domain=1, group_offsets=dev(offs))
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(xb, domain=1, group_offsets=offs)
    assert np.array_equal(host(gsc), rg)
    assert np.array_equal(host(s), rs) and np.array_equal(host(c), rc)


@pytest.mark.parametrize("wid", [0, 2])
def test_expert_weights(wid):
    """a0: per-expert weight quantization of the gate|up and down matrices."""
    w, W1, W2 = moe_case(wid)
    for name, wb, ref in (("w1", w.w1, W1), ("w2", w.w2, W2)):
        say("weights", wid, name, wb.shape)
        from nvfp4_w4a4_quantized_amd.ops import NvFp4Weights
        q = NvFp4Weights.quantize(dev_bf16(wb))
        torch.cuda.synchronize()
        assert np.array_equal(host(q.gscale), ref[2]), name
        assert np.array_equal(host(q.scales), ref[1]), name
        assert np.array_equal(host(q.codes), ref[0]), name


def test_deterministic_repeat():
    w, _, _ = moe_case(2, with_weights=False)
    xd = dev_bf16(w.x)
    a = _ops().nvfp4_quantize(xd)
    b = _ops().nvfp4_quantize(xd)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def _e4m3_midpoint_rows(amax):
    """Rows whose block-scale quotients fl(bmax / fl(6 s_g)) sit exactly on
    E4M3 rounding midpoints, and on the bf16 neighbours of those bmax values.
    amax = 2688 (1536 under Four-Over-Six) makes s_g = 1 and the divisor
    exactly 6; bmax = 6 mu for a midpoint mu needs at most 7 significant
    bits, so it is a bf16 value."""
    mids = []
    for e in range(1, 16):                       # normal binades 2^-6 .. 2^8
        base = 2.0 ** (e - 7)
        for m in range(8):                       # between (e, m) and its successor
            mu = base * (1 + (2 * m + 1) / 16)
            if 6 * mu < 0.98 * amax:
                mids.append(mu)
    mids += [(n + 0.5) / 512 for n in range(8)]  # E4M3 subnormal range ties
    bm = []
    for mu in mids:
        v = np.float32(6 * mu)
        b = int(to_bf16_bits(np.array([v]))[0])
        assert float(np.array([b << 16], np.uint32).view(np.float32)[0]) == v
        bm += [b, b - 1, b + 1]                  # the tie and the neighbouring bf16 values
    rng = np.random.default_rng(41)
    nb = 128
    rows = []
    for r0 in range(0, len(bm), nb - 1):
        chunk = bm[r0:r0 + nb - 1]
        row = np.zeros(16 * nb, np.uint16)
        row[0] = int(to_bf16_bits(np.array([amax], np.float32))[0])
        for i, b in enumerate(chunk):
            blk = 16 * (i + 1)
            bmax = float(np.array([b << 16], np.uint32).view(np.float32)[0])
            # the block maximum in a random slot, smaller random values around it
            vals = rng.uniform(-1, 1, 16).astype(np.float32) * np.float32(bmax * 0.9)
            vals[rng.integers(16)] = bmax * (1 if rng.random() < 0.5 else -1)
            row[blk:blk + 16] = to_bf16_bits(vals)
            row[blk + int(np.argmax(np.abs(vals)))] = b | (0x8000 if vals[np.argmax(np.abs(vals))] < 0 else 0)
        rows.append(row)
    return np.stack(rows)


@pytest.mark.parametrize("rule", [0, 1])
def test_block_scale_quotient_midpoints(rule):
    """The block scale's E4M3 rounding at exact midpoints (ties to even) and
    next to them, through the per-token quantizer, the given-amax block
    quantizer and the routing scatter."""
    amax = 2688.0 if rule == 0 else 1536.0
    xb = _e4m3_midpoint_rows(amax)
    T = xb.shape[0]
    ops = _ops()
    say("block-scale midpoints", rule, xb.shape)
    c, s, g = ops.nvfp4_quantize(dev_bf16(xb), block_rule=rule)
    am = np.full(T, amax, np.float32)
    c2, s2, g2 = ops.nvfp4_quantize(dev_bf16(xb), amax_in=dev(am), block_rule=rule)
    idx = np.zeros((T, 1), np.int32)
    prob = np.ones((T, 1), np.float32)
    p = ops.moe_permute(dev_bf16(xb), dev(idx), dev(prob), 1, block_rule=rule)
    torch.cuda.synchronize()
    rc, rs, rg = O.quantize(xb, rule=rule)
    for what, (hc, hs, hg) in (("per token", (c, s, g)), ("amax_in", (c2, s2, g2)),
                               ("scatter", (p["codes"], p["scales"], p["gscale"]))):
        assert np.array_equal(host(hg).view(np.uint32), rg.view(np.uint32)), what
        hs = host(hs)
        if not np.array_equal(hs, rs):
            r, b = np.argwhere(hs != rs)[0]
            raise AssertionError(f"{what}: scale of row {r} block {b}: gpu {hs[r, b]:02x} "
                                 f"oracle {rs[r, b]:02x}")
        assert np.array_equal(host(hc), rc), what
