"""GPU parity of the paths the C ABI accepts beyond the headline shapes:
more than 128 experts (the router's four-experts-per-lane ranking), K
longer than 4096 in the decode kernels (their K loop is not unrolled),
no clamp (clamp = +inf), a NaN scale byte through the prefill kernels, and
the fused residual add + RMSNorm entry point.  Each case compares the HIP
path, called through the C ABI, with the fp64 oracle on seeded inputs.
"""
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle.workload_inputs import make_inputs
from moe_inputs import synth
from moe_inputs.workloads import WORKLOADS, Workload
import sparse_moe_transformer_softmax_amd as moe
from tests.parity_util import KEYS, TOL, bf16_excess, bf16_tensor_to_f64, check_routing, rel_max_err, to_gpu

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "no GPU"
    moe.lib()
    return _t


def run_and_check(torch, inp, k, clamp, label, sample=None):
    T, d = inp["x"].shape
    E = inp["router_w"].shape[0]
    say(f"{label} T={T} d={d} I={inp['w2_codes'].shape[2] * 2} E={E} k={k} clamp={clamp}")
    g = to_gpu(inp)
    out, out_f32, ids, w, counts = moe.moe_layer_forward_dbg(*[g[kk] for kk in KEYS], k=k, clamp=clamp)
    torch.cuda.synchronize()
    logits, ids_r, w_r = O.route(inp["x"], inp["router_w"], inp["router_b"], k)
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy(), dict(ids=ids_r, w=w_r, logits=logits), E)
    assert torch.equal(out, out_f32.to(torch.bfloat16))
    sel = np.arange(T) if sample is None else np.asarray(sample)
    with np.errstate(over="ignore"):
        ref = O.moe_layer(inp["x"][sel], inp["router_w"], inp["router_b"], inp, k, clamp)["y"]
    o16 = bf16_tensor_to_f64(out)[sel]
    o32 = out_f32.double().cpu().numpy()[sel]
    ex, e32 = bf16_excess(o16, ref), rel_max_err(o32, ref)
    say(f"{label}: excess/rms={ex:.3e} fp32 max/rms={e32:.3e}")
    assert ex <= TOL and e32 <= TOL
    return out


# more than 128 experts: decode sizes (16-row tiles with the folded combine)
# and prefill sizes (128-row tiles)
@pytest.mark.parametrize("T,d,I,E,k", [(40, 128, 64, 200, 8), (64, 64, 32, 256, 8), (2100, 64, 64, 256, 8)])
def test_more_than_128_experts(torch, T, d, I, E, k):
    wl = Workload("wide-e", T=T, d=d, I=I, E=E, k=k, seed=0x5EED5000 + T + E)
    sample = None if T <= 64 else np.sort(np.random.default_rng(E).choice(T, 64, replace=False))
    run_and_check(torch, make_inputs(wl), k, 7.0, f"E={E}", sample)


# K above 4096 in the decode kernels (more than eight 16-block phases): odd
# and even K/32 in the gate/up projection, even K/32 in the down projection,
# 16- and 32-row tiles
@pytest.mark.parametrize("T,d,I,E,k", [(8, 4128, 64, 8, 4), (8, 4160, 64, 8, 4), (8, 64, 4160, 8, 4),
                                       (48, 4160, 64, 8, 4)])
def test_decode_k_above_4096(torch, T, d, I, E, k):
    wl = Workload("long-k", T=T, d=d, I=I, E=E, k=k, seed=0x5EED6000 + T + d + I)
    run_and_check(torch, make_inputs(wl), k, 7.0, f"decode K>4096 d={d} I={I}")


def _stress(inp):
    inp = dict(inp)
    inp["w13_scales"] = ((inp["w13_scales"] - 121) % 3 + 127).astype(np.uint8)
    inp["w2_scales"] = ((inp["w2_scales"] - 121) % 3 + 127).astype(np.uint8)
    return inp


@pytest.mark.parametrize("stress", [False, True], ids=["plain", "large-preact"])
def test_no_clamp_tiny(torch, stress):
    """clamp = +inf: the activation is Swish(g) * (u + 1) with no limit; the
    large-preactivation variant (scale exponents 0..2) drives |g| past 60,
    where exp overflows and the sigmoid is exactly 0 or 1."""
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    run_and_check(torch, _stress(inp) if stress else inp, wl.k, float("inf"), f"tiny no clamp stress={stress}")


def test_no_clamp_prefill(torch):
    wl = Workload("noclamp", T=1500, d=256, I=192, E=8, k=3, seed=0x5EED7000)
    sample = np.sort(np.random.default_rng(5).choice(wl.T, 64, replace=False))
    run_and_check(torch, _stress(make_inputs(wl)), wl.k, float("inf"), "prefill no clamp", sample)


@pytest.mark.parametrize("d,I", [(256, 192), (288, 96)], ids=["128-row-tiles", "64-row-tiles"])
def test_nan_scale_propagates_at_prefill(torch, d, I):
    """A NaN scale byte (0xFF) in a gate row makes every output of the
    tokens routed to that expert NaN; one in a down row makes that output
    column NaN for the tokens of its expert."""
    wl = Workload("nan-prefill", T=1500, d=d, I=I, E=8, k=3, seed=0x5EED8000 + d)
    inp = dict(make_inputs(wl))
    inp["w13_scales"] = inp["w13_scales"].copy()
    inp["w2_scales"] = inp["w2_scales"].copy()
    inp["w13_scales"][3, 5, 1] = 0xFF
    inp["w2_scales"][5, 7, 2] = 0xFF
    say(f"nan scale prefill d={d} I={I}")
    g = to_gpu(inp)
    out = moe.moe_layer_forward(*[g[kk] for kk in KEYS], k=wl.k, clamp=wl.clamp)
    torch.cuda.synchronize()
    ref = O.moe_layer(inp["x"], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp)["y"]
    nan_ref = np.isnan(ref)
    nan_gpu = torch.isnan(out.float()).cpu().numpy()
    assert nan_ref.any(axis=1).sum() > 100 and (nan_ref.all(axis=1).sum() < nan_ref.any(axis=1).sum())
    assert np.array_equal(nan_ref, nan_gpu)
    fin = ~nan_ref
    assert bf16_excess(bf16_tensor_to_f64(out)[fin], ref[fin]) <= TOL


# ---------------------------------------------------------------------------
# residual add + RMSNorm between stack layers
# ---------------------------------------------------------------------------

def _bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("y_dtype", ["f32", "bf16"])
def test_rmsnorm_residual(torch, y_dtype):
    """x_out equals torch's fp32 add rounded to bf16 bit for bit; n_out
    equals the library's own RMSNorm of x_out bit for bit and the oracle's
    RMSNorm within bf16 rounding; in place (x_out = x) gives the same."""
    rng = np.random.default_rng(17)
    T, d = 77, 2880
    x = _bf16(torch, synth.f32_to_bf16_bits((rng.standard_normal((T, d)) * 40).astype(np.float32)))
    yf = torch.from_numpy((rng.standard_normal((T, d)) * 30).astype(np.float32)).cuda()
    y = yf if y_dtype == "f32" else yf.to(torch.bfloat16)
    say(f"rmsnorm_residual y={y_dtype}")
    xo, no = moe.moe_rmsnorm_residual(x, y, 1e-5)
    want_x = (x.float() + y.float()).to(torch.bfloat16)
    want_n = moe.moe_rmsnorm(want_x, 1e-5)
    x2 = x.clone()
    xo2, no2 = moe.moe_rmsnorm_residual(x2, y, 1e-5, x_out=x2)
    xo3, none = moe.moe_rmsnorm_residual(x, y, 1e-5, normalize=False)
    torch.cuda.synchronize()
    assert torch.equal(xo, want_x) and torch.equal(no, want_n)
    assert torch.equal(xo2, want_x) and torch.equal(no2, want_n) and xo2.data_ptr() == x2.data_ptr()
    assert torch.equal(xo3, want_x) and none is None
    ref = O.rmsnorm(bf16_tensor_to_f64(xo), 1e-5)
    assert bf16_excess(bf16_tensor_to_f64(no), ref) <= 1e-5
