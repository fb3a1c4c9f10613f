"""Pins of the fp64 oracle against facts that do not come from the oracle:
the OCP E2M1 table, closed forms, library routines, invariants, brute force.

Each test names the mistake it is there to catch.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from moe_inputs import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------
# MXFP4 decode
# --------------------------------------------------------------------------

def test_e2m1_codes_match_ocp_table():
    """All 16 codes against the OCP MX table (catches a wrong exponent bias,
    a subnormal mistake or a sign-bit position error)."""
    table = {int(c): float(v) for c, v in _golden("e2m1_codes.txt")}
    got = O.e2m1_value(np.arange(16))
    for c in range(16):
        assert got[c] == table[c], c
        assert math.copysign(1.0, got[c]) == math.copysign(1.0, table[c]), c


def test_e8m0_every_byte():
    """2^(s-127) for all 255 finite bytes, NaN for 0xFF (catches a bias
    off by one)."""
    v = O.e8m0_value(np.arange(256))
    for s in range(255):
        assert v[s] == math.ldexp(1.0, s - 127)
    assert math.isnan(v[255])


def test_mxfp4_all_codes_times_all_scales():
    """16 codes x 256 scale bytes decode to code-value * 2^(s-127)."""
    table = {int(c): float(v) for c, v in _golden("e2m1_codes.txt")}
    R = 256
    K = 32
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    for j in range(K // 2):
        lo, hi = (2 * j) % 16, (2 * j + 1) % 16
        codes[:, j] = lo | (hi << 4)
    scales = np.arange(256, dtype=np.uint8).reshape(R, 1)
    w = O.mxfp4_dequant(codes, scales)
    for s in range(256):
        for i in range(K):
            c = i % 16
            if s == 255:
                assert math.isnan(w[s, i])
            else:
                assert w[s, i] == table[c] * math.ldexp(1.0, s - 127), (s, i)


def test_mxfp4_nibble_order_and_block_index():
    """Element 2j is the low nibble, 2j+1 the high nibble; scale byte b
    covers elements [32b, 32b+32) (catches swapped nibbles and a scale
    indexed per 16 or per row)."""
    K = 96
    rng = np.random.default_rng(1)
    lo = rng.integers(0, 16, K // 2)
    hi = rng.integers(0, 16, K // 2)
    codes = (lo | (hi << 4)).astype(np.uint8)[None, :]
    scales = np.array([[127, 130, 120]], dtype=np.uint8)
    w = O.mxfp4_dequant(codes, scales)[0]
    table = {int(c): float(v) for c, v in _golden("e2m1_codes.txt")}
    for i in range(K):
        code = lo[i // 2] if i % 2 == 0 else hi[i // 2]
        assert w[i] == table[int(code)] * math.ldexp(1.0, int(scales[0, i // 32]) - 127)


def test_format_sizes_match_pages():
    """4.25 bits per weight, and the checkpoint sizes the pages print follow
    from d = I = 2880, a 3-matrix GLU, the expert and block counts, with the
    remaining parameters in bf16 (catches a wrong expert shape or format)."""
    g = {r[0]: float(r[1]) for r in _golden("page_sizes.txt")}
    assert (32 * 4 + 8) / 32 == g["bits_per_weight"]
    d, I = int(g["d_model"]), int(g["expert_width"])
    per_expert = 3 * d * I
    # MXFP4 bytes of one expert at d = I = 2880
    assert per_expert * 4.25 / 8 == 13_219_200
    for tag, E, L, P in (("120b", g["experts_120b"], g["blocks_120b"], g["params_120b"]),
                         ("20b", g["experts_20b"], g["blocks_20b"], g["params_20b"])):
        moe = L * E * per_expert
        rest = P - moe
        gib = (moe * g["bits_per_weight"] / 8 + rest * 2) / 2**30
        assert abs(gib / g[f"ckpt_gib_{tag}"] - 1) < 0.02, (tag, gib)


# --------------------------------------------------------------------------
# bf16 helpers
# --------------------------------------------------------------------------

def test_bf16_decode_and_round_match_torch():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    bits = synth.f32_to_bf16_bits(v)
    tb = torch.from_numpy(v).to(torch.bfloat16)
    assert np.array_equal(bits, tb.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(O.bf16_bits_to_f64(bits), tb.to(torch.float64).numpy())
    assert np.array_equal(O.round_to_bf16(v.astype(np.float64)), tb.to(torch.float64).numpy())


# --------------------------------------------------------------------------
# router, top-k, softmax
# --------------------------------------------------------------------------

def _tiny_router(T=64, d=64, E=8, seed=3):
    x = synth.gen_x(seed, T, d)
    wr, br = synth.gen_router(seed, E, d)
    return x, wr, br


def test_gate_weights_sum_to_one():
    x, wr, br = _tiny_router()
    for k in (1, 2, 4, 8):
        _, ids, w = O.route(x, wr, br, k)
        assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-15)
        if k == 1:
            assert np.all(w == 1.0)


def test_k_equals_E_is_full_softmax():
    """Selecting every expert reduces to the textbook softmax (catches a
    sign error in the exponent or a missing max shift)."""
    x, wr, br = _tiny_router()
    logits, ids, w = O.route(x, wr, br, 8)
    full = scipy.special.softmax(logits, axis=1)
    assert np.allclose(np.take_along_axis(full, ids, 1), w, rtol=1e-14, atol=0)


def test_selected_softmax_equals_renormalised_full_softmax():
    x, wr, br = _tiny_router()
    logits, ids, w = O.route(x, wr, br, 4)
    full = scipy.special.softmax(logits, axis=1)
    sel = np.take_along_axis(full, ids, 1)
    assert np.allclose(sel / sel.sum(1, keepdims=True), w, rtol=1e-13, atol=0)


def test_topk_brute_force_over_all_subsets():
    """The selected set maximises the summed logit over all C(8,4) = 70
    subsets; slots are in descending logit order (catches ascending order
    or an off-by-one in k)."""
    x, wr, br = _tiny_router(T=200)
    logits, ids, _ = O.route(x, wr, br, 4)
    for t in range(logits.shape[0]):
        best = max(itertools.combinations(range(8), 4), key=lambda s: sum(logits[t, list(s)]))
        assert set(best) == set(ids[t].tolist())
        assert np.all(np.diff(logits[t, ids[t]]) <= 0)


def test_topk_ties_go_to_lower_index():
    lg = np.zeros((3, 8))
    lg[1, [2, 5, 6]] = 1.0
    lg[2] = [0, 3, 3, 1, 3, 2, 3, 0]
    ids = O.topk_experts(lg, 4)
    assert ids[0].tolist() == [0, 1, 2, 3]
    assert ids[1].tolist() == [2, 5, 6, 0]
    assert ids[2].tolist() == [1, 2, 4, 6]


def test_topk_gap_against_subset_brute_force():
    """The gap of a row is the distance from the weakest selected logit to
    the strongest unselected one, the selected set taken by brute force over
    all C(8,4) = 70 subsets; moving those two logits towards each other by
    half the gap plus a little changes the set, any perturbation below half
    the gap keeps it (catches the gap between slots k-2 and k-1, a sign
    error, or a gap measured from the wrong end of the order)."""
    x, wr, br = _tiny_router(T=120)
    logits, _, _ = O.route(x, wr, br, 4)
    gap = O.topk_gap(logits, 4)
    rng = np.random.default_rng(4)
    for t in range(logits.shape[0]):
        l = logits[t]
        best = max(itertools.combinations(range(8), 4), key=lambda s: sum(l[list(s)]))
        rest = [e for e in range(8) if e not in best]
        want = min(l[list(best)]) - max(l[rest])
        assert gap[t] == want
        assert gap[t] > 0
        lo = min(best, key=lambda e: l[e])
        hi = max(rest, key=lambda e: l[e])
        moved = l.copy()
        moved[lo] -= 0.5 * gap[t] * 1.01
        moved[hi] += 0.5 * gap[t] * 1.01
        assert hi in O.topk_experts(moved[None, :], 4)[0]
        noise = rng.uniform(-0.49, 0.49, 8) * gap[t]
        assert set(O.topk_experts((l + noise)[None, :], 4)[0]) == set(best)
    # k = E: no unselected expert; a tie at the boundary: gap 0
    assert np.all(np.isinf(O.topk_gap(logits, 8)))
    tie = np.array([[3.0, 1.0, 2.0, 2.0, 0.5]])
    assert O.topk_gap(tie, 2)[0] == 0.0 and O.topk_gap(tie, 1)[0] == 1.0 and O.topk_gap(tie, 3)[0] == 1.0


def test_router_one_hot_input():
    """x = e_j makes each logit W_r[e, j] + b[e] (catches a transposed
    router weight or a dropped bias)."""
    d, E = 64, 8
    wr, br = synth.gen_router(5, E, d)
    for j in (0, 17, 63):
        x = np.zeros((1, d), dtype=np.uint16)
        x[0, j] = 0x3F80  # bf16 1.0
        logits, _, _ = O.route(x, wr, br, 4)
        want = O.bf16_bits_to_f64(wr[:, j]) + br.astype(np.float64)
        assert np.array_equal(logits[0], want)


# --------------------------------------------------------------------------
# experts
# --------------------------------------------------------------------------

def _mx_identity_like(perm, scale_byte=127):
    """MXFP4 encoding of a permutation matrix M[r, perm[r]] = 1."""
    n = len(perm)
    codes = np.zeros((n, n // 2), dtype=np.uint8)
    for r, c in enumerate(perm):
        codes[r, c // 2] |= (2 << 4) if c % 2 else 2      # code 2 = 1.0
    scales = np.full((n, n // 32), scale_byte, dtype=np.uint8)
    return codes, scales


def _experts_from(E, w13c, w13s, b13, w2c, w2s, b2):
    return dict(w13_codes=np.stack([w13c] * E), w13_scales=np.stack([w13s] * E),
                b13=np.stack([b13] * E).astype(np.float32), w2_codes=np.stack([w2c] * E),
                w2_scales=np.stack([w2s] * E), b2=np.stack([b2] * E).astype(np.float32))


def test_identical_experts_reduce_to_one_ffn():
    """With all experts equal, any routing gives the single-expert FFN
    because the gate weights sum to one (catches unnormalised weights)."""
    T, d, I, E = 24, 64, 96, 8
    x, wr, br = _tiny_router(T=T, d=d, E=E, seed=7)
    ex = synth.gen_experts(7, 1, d, I)
    ex8 = _experts_from(E, ex["w13_codes"][0], ex["w13_scales"][0], ex["b13"][0],
                        ex["w2_codes"][0], ex["w2_scales"][0], ex["b2"][0])
    y = O.moe_layer(x, wr, br, ex8, 4, 7.0)["y"]
    w13 = O.mxfp4_dequant(ex["w13_codes"][0], ex["w13_scales"][0])
    w2 = O.mxfp4_dequant(ex["w2_codes"][0], ex["w2_scales"][0])
    z = O.expert_ffn(O.bf16_bits_to_f64(x), w13, ex["b13"][0].astype(np.float64), w2,
                     ex["b2"][0].astype(np.float64), 7.0)
    assert np.allclose(y, z, rtol=1e-13, atol=1e-12)


def test_zero_gate_gives_weighted_down_bias():
    """W_gate = 0, b_gate = 0 makes h = 0, so y_t = sum_j w_tj b2[S_tj]
    (catches b2 outside the expert or unweighted)."""
    T, d, I, E = 16, 64, 64, 8
    x, wr, br = _tiny_router(T=T, d=d, E=E, seed=8)
    ex = synth.gen_experts(8, E, d, I)
    ex["w13_codes"][:, :I, :] = 0
    ex["b13"][:, :I] = 0
    r = O.moe_layer(x, wr, br, ex, 4, 7.0)
    want = np.einsum("tj,tjd->td", r["w"], ex["b2"].astype(np.float64)[r["ids"]])
    assert np.allclose(r["y"], want, rtol=1e-14, atol=1e-15)


def test_swish_path_with_permutations_and_clamp():
    """W_gate = P, W_up = 0, W_2 = Q (permutations), zero biases: the layer
    is Q silu(clamp(P x)) -- torch's silu is the library Swish.  Catches a
    transposed W13 or W2, gate/up halves swapped, a wrong clamp."""
    T, d, E, c = 16, 64, 8, 7.0
    I = d
    rng = np.random.default_rng(9)
    P = rng.permutation(I)
    Q = rng.permutation(d)
    x = synth.f32_to_bf16_bits((rng.standard_normal((T, d)) * 6).astype(np.float32))
    wr, br = synth.gen_router(9, E, d)
    gc, gs = _mx_identity_like(P)
    w13c = np.concatenate([gc, np.zeros_like(gc)])
    w13s = np.concatenate([gs, gs])
    w2c, w2s = _mx_identity_like(Q)
    ex = _experts_from(E, w13c, w13s, np.zeros(2 * I), w2c, w2s, np.zeros(d))
    y = O.moe_layer(x, wr, br, ex, 4, c)["y"]
    xf = torch.from_numpy(O.bf16_bits_to_f64(x))
    g = xf[:, P]                                         # (P x)_r = x[P[r]]
    h = torch.nn.functional.silu(g.clamp(-c, c))
    want = h[:, Q].numpy()
    assert np.allclose(y, want, rtol=1e-13, atol=1e-13)
    # saturation: past the clamp the output is exactly silu(c)
    sat = np.abs(xf[:, P].numpy()) > c
    assert sat.any()
    silu_c = c / (1 + math.exp(-c))
    hh = O.clamped_swiglu(xf.numpy()[:, P], np.zeros((T, I)), c)
    assert np.allclose(np.abs(hh[sat]), np.where(xf.numpy()[:, P][sat] > 0, silu_c,
                                                 c / (1 + math.exp(c))), rtol=1e-15)


def test_up_branch_has_plus_one_and_clamp():
    """W_gate = 0 with b_gate = beta, W_up = P: h = silu(beta)(clamp(Px)+1)
    (catches a missing +1 or an unclamped up branch)."""
    T, d, E, c, beta = 16, 64, 8, 7.0, 1.25
    I = d
    rng = np.random.default_rng(10)
    P = rng.permutation(I)
    x = synth.f32_to_bf16_bits((rng.standard_normal((T, d)) * 6).astype(np.float32))
    wr, br = synth.gen_router(10, E, d)
    uc_, us_ = _mx_identity_like(P)
    w13c = np.concatenate([np.zeros_like(uc_), uc_])
    w13s = np.concatenate([us_, us_])
    ic, is_ = _mx_identity_like(np.arange(d))
    b13 = np.concatenate([np.full(I, beta), np.zeros(I)])
    ex = _experts_from(E, w13c, w13s, b13, ic, is_, np.zeros(d))
    y = O.moe_layer(x, wr, br, ex, 4, c)["y"]
    u = O.bf16_bits_to_f64(x)[:, P]
    sb = float(torch.nn.functional.silu(torch.tensor(beta, dtype=torch.float64)))
    assert np.allclose(y, sb * (np.clip(u, -c, c) + 1.0), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("stress", [False, True])
def test_dense_masked_equals_sparse_tiny(stress):
    """Brute force over every expert with a masked mixture equals the sparse
    layer on the tiny workload (T16 d128 I128 E8 k4), and on a clamp-stress
    variant whose scale exponents are 0..2 (pre-activations hit the clamp)."""
    from oracle.workload_inputs import make_inputs
    from moe_inputs.workloads import WORKLOADS
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    if stress:
        inp["w13_scales"] = (inp["w13_scales"] - 121 + 127).astype(np.uint8) % 3 + 127
        inp["w2_scales"] = (inp["w2_scales"] - 121 + 127).astype(np.uint8) % 3 + 127
    r = O.moe_layer(inp["x"], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp)
    yd = O.moe_layer_dense_masked(inp["x"], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp)
    rms = np.sqrt(np.mean(r["y"] ** 2))
    assert np.max(np.abs(r["y"] - yd)) <= 1e-12 * rms
    if stress:
        w13 = O.mxfp4_dequant(inp["w13_codes"][0], inp["w13_scales"][0])
        a = O.bf16_bits_to_f64(inp["x"]) @ w13.T
        assert np.mean(np.abs(a) > wl.clamp) > 0.2


# --------------------------------------------------------------------------
# RMSNorm and the residual stack
# --------------------------------------------------------------------------

def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(11)
    v = rng.standard_normal((8, 2880)) * 30
    want = torch.nn.functional.rms_norm(torch.from_numpy(v), (2880,), eps=1e-5).numpy()
    assert np.allclose(O.rmsnorm(v, 1e-5), want, rtol=1e-14, atol=0)
    c = np.full((1, 32), 3.0)
    assert np.allclose(O.rmsnorm(c, 1e-5), 3.0 / math.sqrt(9.0 + 1e-5), rtol=1e-15)


def test_stack_constant_down_bias_is_a_shift():
    """Zero gate/up weights and biases with b2 = const make every layer add
    exactly that constant (weights sum to one): x_L = bf16(...bf16(x0 + c)...)."""
    T, d, I, E, L, c = 8, 64, 32, 8, 3, 0.75
    x0 = synth.gen_x(12, T, d)
    layers = []
    for l in range(L):
        ex = synth.gen_experts(100 + l, E, d, I)
        ex["w13_codes"][:] = 0
        ex["b13"][:] = 0
        ex["b2"][:] = c
        wr, br = synth.gen_router(100 + l, E, d)
        ex.update(router_w=wr, router_b=br)
        layers.append(ex)
    x, _ = O.stack_forward(x0, layers, 4, 7.0)
    want = O.bf16_bits_to_f64(x0)
    for _ in range(L):
        want = torch.from_numpy(want + c).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(x, want)
