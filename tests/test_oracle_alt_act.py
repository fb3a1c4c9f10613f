"""Pins of the variant activation reading (CPU): Swish with slope 1.702 on
the gate clamped from above only, the up branch clamped on both sides, and
gate/up rows interleaved in the fused weight.  Checked against torch's SiLU
(a library routine), closed forms at the clamp, and layouts that only the
interleaved reading maps to the expected output."""
import numpy as np
import torch

from oracle import moe_oracle as O
from oracle.workload_inputs import make_inputs
from moe_inputs.workloads import WORKLOADS


def test_alt_swish_is_scaled_silu():
    # v * sigmoid(a v) = silu(a v) / a
    g = np.linspace(-6.5, 6.5, 201)
    u = np.zeros_like(g)
    a = O.ALT_SWISH_SLOPE
    want = torch.nn.functional.silu(torch.tensor(a * g, dtype=torch.float64)).numpy() / a
    assert np.allclose(O.clamped_swiglu_alt(g, u, 7.0), want, rtol=1e-13, atol=1e-15)


def test_alt_clamps():
    c = 7.0
    a = O.ALT_SWISH_SLOPE
    # gate clamped from above only
    h_hi = O.clamped_swiglu_alt(np.array([100.0]), np.array([0.0]), c)[0]
    assert np.isclose(h_hi, c / (1 + np.exp(-a * c)), rtol=1e-14)
    g_lo = -30.0
    h_lo = O.clamped_swiglu_alt(np.array([g_lo]), np.array([0.0]), c)[0]
    assert np.isclose(h_lo, g_lo / (1 + np.exp(-a * g_lo)), rtol=1e-12)
    # up clamped on both sides, then + 1
    for u, uc in [(50.0, c), (-50.0, -c), (3.0, 3.0)]:
        h = O.clamped_swiglu_alt(np.array([1.0]), np.array([u]), c)[0]
        assert np.isclose(h, (1.0 / (1 + np.exp(-a))) * (uc + 1.0), rtol=1e-14)


def test_alt_layout_zero_gate_rows_give_the_down_bias():
    # zero every even (gate) row of W13 and every even b13 entry: with the
    # interleaved reading h = 0, so each token's output is sum_j w_j b2 = b2
    # of a common down bias; the gate-first reading would see the odd rows
    # in its gate half and give something else
    wl = WORKLOADS["tiny"]
    inp = dict(make_inputs(wl))
    codes = inp["w13_codes"].copy()
    codes[:, 0::2, :] = 0  # E2M1 code 0 = +0
    b13 = inp["b13"].copy()
    b13[:, 0::2] = 0.0
    b2 = np.tile(np.linspace(-1, 1, wl.d, dtype=np.float32), (wl.E, 1))
    inp.update(w13_codes=codes, b13=b13, b2=b2)
    args = (inp["x"], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp)
    y_alt = O.moe_layer(*args, alt=True)["y"]
    assert np.allclose(y_alt, np.tile(b2[0].astype(np.float64), (wl.T, 1)), rtol=0, atol=1e-12)
    y_std = O.moe_layer(*args)["y"]
    assert np.abs(y_std - y_alt).max() > 1e-3


def test_alt_layout_equals_standard_on_permuted_rows_when_activations_agree():
    # with |gate| and |up| inside the clamp and the activation slope set to
    # one, the interleaved layout is the gate-first layout with its rows
    # permuted; check that reading through expert_ffn on one expert
    rng = np.random.default_rng(11)
    d, I = 64, 32
    xs = rng.standard_normal((5, d)) * 0.1
    w13 = rng.standard_normal((2 * I, d)) * 0.05
    b13 = rng.standard_normal(2 * I) * 0.01
    w2 = rng.standard_normal((d, I)) * 0.05
    b2 = rng.standard_normal(d) * 0.01
    perm = np.empty(2 * I, dtype=int)
    perm[0::2] = np.arange(I)
    perm[1::2] = I + np.arange(I)
    slope = O.ALT_SWISH_SLOPE
    try:
        O.ALT_SWISH_SLOPE = 1.0
        z_alt = O.expert_ffn(xs, w13[perm], b13[perm], w2, b2, 7.0, None, True)
    finally:
        O.ALT_SWISH_SLOPE = slope
    z_std = O.expert_ffn(xs, w13, b13, w2, b2, 7.0)
    assert np.allclose(z_alt, z_std, rtol=1e-13, atol=1e-15)
