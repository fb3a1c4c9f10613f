"""Pins of the two-term activation option's oracle piece (CPU):
mx6x2_quantize against brute force over the E2M3 grid term by term, the
error bound that follows from the scale rule, and the layer's deviation
from the exact layer against the one-term fast mode's."""
import numpy as np

from oracle import moe_oracle as O
from oracle.workload_inputs import make_inputs
from moe_inputs.workloads import WORKLOADS
from tests.test_oracle_mxfp6 import brute_round, e2m3_grid


def _blocks(seed, rows=4, nblk=3):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, 32 * nblk)) * np.exp2(rng.integers(-10, 10, (rows, 1)))
    # a few blocks with a wide spread of magnitudes, and one all-zero block
    v[0, :32] *= np.exp2(rng.integers(-12, 0, 32))
    v[1, 32:64] = 0.0
    return v


def _brute_term(blk):
    """One MXFP6 term of a block by brute force: the scale 2^k with k the
    smallest integer such that 7.5 2^k covers the block's largest magnitude,
    then the nearest grid value of each element (ties to the even code)."""
    amax = float(np.abs(blk).max())
    if amax == 0.0:
        return np.zeros_like(blk)
    k = -127
    while 7.5 * 2.0 ** k < amax:
        k += 1
    s = 2.0 ** k
    return np.array([brute_round(x / s) for x in blk]) * s


def test_two_terms_are_brute_force_terms():
    v = _blocks(11)
    q = O.mx6x2_quantize(v)
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, 32 * b:32 * b + 32]
            t0 = _brute_term(blk)
            t1 = _brute_term(blk - t0)
            assert np.array_equal(q[r, 32 * b:32 * b + 32], t0 + t1)


def test_two_term_error_bound():
    # the scale rule gives s < amax / 3.75 and E2M3 rounds to within a
    # quarter of the scale, so one term leaves less than amax / 15 and two
    # terms less than amax / 225 (of the block's largest magnitude)
    for seed in range(5):
        v = _blocks(100 + seed, rows=8, nblk=4)
        q1, q2 = O.mxfp6_quantize(v), O.mx6x2_quantize(v)
        b = v.reshape(v.shape[0], -1, 32)
        amax = np.abs(b).max(axis=-1)
        e1 = np.abs(b - q1.reshape(b.shape)).max(axis=-1)
        e2 = np.abs(b - q2.reshape(b.shape)).max(axis=-1)
        live = amax > 0
        assert np.all(e1[live] < amax[live] / 15)
        assert np.all(e2[live] < amax[live] / 225)
        assert np.all(e2[live] < e1[live] / 15 + 1e-300)
        assert np.all(e2[~live] == 0)


def test_one_term_values_are_kept():
    v = O.mxfp6_quantize(_blocks(21))
    assert np.array_equal(O.mx6x2_quantize(v), v)


def test_second_term_sits_on_its_own_grid():
    v = _blocks(31)
    t0 = O.mxfp6_quantize(v)
    t1 = O.mx6x2_quantize(v) - t0
    grid = np.array([w for w, _ in e2m3_grid()])
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            res = v[r, 32 * b:32 * b + 32] - t0[r, 32 * b:32 * b + 32]
            amax = np.abs(res).max()
            if amax == 0:
                continue
            s = 2.0 ** O.mx6_scale_exponent(amax)
            assert np.all(np.isin(np.abs(t1[r, 32 * b:32 * b + 32]) / s, grid))


def test_two_term_layer_deviates_far_less_than_one_term():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    args = (inp["x"], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp)
    ex = O.moe_layer(*args)
    one = O.moe_layer(*args, act="mxfp6")
    two = O.moe_layer(*args, act="mx6x2")
    assert np.array_equal(ex["ids"], two["ids"]) and np.array_equal(ex["w"], two["w"])
    rms = np.sqrt((ex["y"] ** 2).mean())
    d1 = np.sqrt(((one["y"] - ex["y"]) ** 2).mean()) / rms
    d2 = np.sqrt(((two["y"] - ex["y"]) ** 2).mean()) / rms
    assert 0 < d2 < d1 / 5, (d1, d2)
