"""Pins of the activation-quantised fast mode's oracle pieces (CPU): the
FP6 E2M3 rounding, the per-block scale rule and the MXFP6 quantiser, each
checked against brute force over the format's own grid, and the fast-mode
layer's wiring through its size of deviation from the exact layer."""
import itertools

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle.workload_inputs import make_inputs
from moe_inputs.workloads import WORKLOADS


def e2m3_grid():
    """All non-negative E2M3 values with their codes, from the format's
    definition (bias 1; e = 0: m/8; e >= 1: 2^(e-1) (1 + m/8))."""
    out = []
    for e, m in itertools.product(range(4), range(8)):
        v = m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0)
        out.append((v, (e << 3) | m))
    return out


def brute_round(v):
    """Nearest grid value; on a tie the one whose code is even."""
    g = e2m3_grid()
    a = abs(v)
    best = min(g, key=lambda t: (abs(t[0] - a), t[1] & 1))
    return np.copysign(best[0], v)


def test_e2m3_grid_is_fixed_and_ordered():
    g = e2m3_grid()
    vals = [v for v, _ in g]
    assert vals == sorted(vals) and len(set(vals)) == 32
    assert vals[-1] == 7.5 and vals[1] == 0.125 and vals[8] == 1.0
    for v, _ in g:
        assert O.e2m3_round(np.array([v]))[0] == v
        assert O.e2m3_round(np.array([-v]))[0] == -v


def test_e2m3_round_matches_brute_force_incl_every_midpoint():
    g = [v for v, _ in e2m3_grid()]
    mids = [(a + b) / 2 for a, b in zip(g[:-1], g[1:])]
    rng = np.random.default_rng(3)
    vals = np.concatenate([mids, -np.array(mids), rng.uniform(-7.5, 7.5, 2000)])
    got = O.e2m3_round(vals)
    want = np.array([brute_round(v) for v in vals])
    assert np.array_equal(got, want)


def test_scale_exponent_is_the_smallest_covering_power():
    rng = np.random.default_rng(4)
    amax = np.concatenate([np.exp2(rng.uniform(-30, 30, 500)), 7.5 * np.exp2(np.arange(-20, 20)),
                           np.nextafter(7.5 * np.exp2(np.arange(-20, 20)), np.inf)])
    k = O.mx6_scale_exponent(amax)
    for a, kk in zip(amax, k):
        assert 7.5 * 2.0 ** kk >= a and 7.5 * 2.0 ** (kk - 1) < a
    assert O.mx6_scale_exponent(np.array([0.0]))[0] == -127


def test_mxfp6_blocks_lie_on_their_grid_and_are_nearest():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((3, 96)) * np.exp2(rng.integers(-8, 8, (3, 1)))
    q = O.mxfp6_quantize(v)
    grid = np.array([w for w, _ in e2m3_grid()])
    for r in range(3):
        for b in range(3):
            blk, qb = v[r, 32 * b:32 * b + 32], q[r, 32 * b:32 * b + 32]
            k = O.mx6_scale_exponent(np.abs(blk).max())
            s = 2.0 ** k
            # every element is a scaled grid value, the nearest one to it
            assert np.all(np.isin(np.abs(qb) / s, grid))
            assert np.array_equal(qb, np.array([brute_round(x / s) for x in blk]) * s)
    assert np.array_equal(O.mxfp6_quantize(q), q)  # idempotent
    assert np.array_equal(O.mxfp6_quantize(np.zeros((1, 32))), np.zeros((1, 32)))


def test_fast_mode_layer_deviates_like_a_six_bit_activation():
    # the fast mode differs from the exact layer by the activation rounding
    # alone: an rms deviation of a few per cent (three mantissa bits, plus
    # the coarse subnormal step for values far below their block maximum),
    # never zero (the rounding is applied) and never of order one (it is
    # applied to x and h, not to the weights or outputs); the routing is
    # the same
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    args = (inp["x"], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp)
    ex = O.moe_layer(*args)
    fa = O.moe_layer(*args, act="mxfp6")
    assert np.array_equal(ex["ids"], fa["ids"]) and np.array_equal(ex["w"], fa["w"])
    rms = np.sqrt((ex["y"] ** 2).mean())
    dev_rms = np.sqrt(((fa["y"] - ex["y"]) ** 2).mean()) / rms
    dev_max = np.abs(fa["y"] - ex["y"]).max() / rms
    assert 5e-3 < dev_rms < 0.15, dev_rms
    assert dev_max < 0.6, dev_max


def test_fast_mode_rejects_unknown_modes():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    with pytest.raises(ValueError):
        O.moe_layer(inp["x"], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp, act="fp8")
