"""GPU parity of the variant activation reading (moe_layer_forward_ex with
MOE_LAYER_ALT_ACT: interleaved gate/up rows, Swish slope 1.702, gate clamped
from above only) against the oracle's alt=True layer, on the same raw
arrays read the variant way by both sides; also combined with the fast mode.
Same bars as the exact path: routing exact, outputs within
max|err| <= 1e-2 * rms(ref) beyond the final bf16 rounding."""
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle.workload_inputs import make_inputs
from moe_inputs.workloads import WORKLOADS, Workload
import sparse_moe_transformer_softmax_amd as moe
from tests.parity_util import TOL, KEYS, bf16_excess, bf16_tensor_to_f64, check_routing, rel_max_err, to_gpu

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


def run_alt(torch, inp, k, clamp, flags, sample=None, label=""):
    E = inp["router_w"].shape[0]
    T = inp["x"].shape[0]
    say(f"alt {label} flags={flags} T={T} d={inp['x'].shape[1]} I={inp['w2_codes'].shape[2] * 2} E={E} k={k}")
    g = to_gpu(inp)
    out, out_f32, ids, w, counts = moe.moe_layer_forward_ex(*[g[kk] for kk in KEYS], k=k, clamp=clamp,
                                                            flags=flags, debug=True)
    torch.cuda.synchronize()
    logits, ids_r, w_r = O.route(inp["x"], inp["router_w"], inp["router_b"], k)
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy(),
                  dict(ids=ids_r, w=w_r, logits=logits), E)
    assert torch.equal(out, out_f32.to(torch.bfloat16))
    sel = np.arange(T) if sample is None else np.asarray(sample)
    act = "mxfp6" if flags & moe.MOE_LAYER_MXFP6 else "exact"
    ref = O.moe_layer(inp["x"][sel], inp["router_w"], inp["router_b"], inp, k, clamp, act=act, alt=True)["y"]
    o16 = bf16_tensor_to_f64(out)[sel]
    o32 = out_f32.double().cpu().numpy()[sel]
    ex, e32 = bf16_excess(o16, ref), rel_max_err(o32, ref)
    say(f"alt {label}: excess/rms={ex:.3e} fp32 max/rms={e32:.3e}")
    assert ex <= TOL and e32 <= TOL


ALT = moe.MOE_LAYER_ALT_ACT


def test_alt_tiny(torch):
    wl = WORKLOADS["tiny"]
    run_alt(torch, make_inputs(wl), wl.k, wl.clamp, ALT, label="tiny")


def test_alt_tiny_clamp_stress(torch):
    # scale exponents 0..2: gate and up pre-activations reach far past the
    # clamp on both sides (the gate's lower side is left unclamped)
    wl = WORKLOADS["tiny"]
    inp = dict(make_inputs(wl))
    inp["w13_scales"] = ((inp["w13_scales"] - 121) % 3 + 127).astype(np.uint8)
    inp["w2_scales"] = ((inp["w2_scales"] - 121) % 3 + 127).astype(np.uint8)
    run_alt(torch, inp, wl.k, wl.clamp, ALT, label="tiny-clamp-stress")


def test_alt_decode_20b(torch):
    wl = WORKLOADS["20b_decode"]
    run_alt(torch, make_inputs(wl), wl.k, wl.clamp, ALT, label="20b-decode")


def test_alt_prefill_20b_sampled(torch):
    wl = WORKLOADS["20b_prefill"]
    rng = np.random.default_rng(27)
    sample = np.sort(rng.choice(wl.T, 40, replace=False))
    run_alt(torch, make_inputs(wl), wl.k, wl.clamp, ALT, sample=sample, label="20b-prefill")


@pytest.mark.parametrize("T,d,I,E,k", [
    (37, 160, 96, 24, 2),    # 16-row decode tiles, K/32 odd
    (300, 128, 128, 16, 1),  # 32-row decode tiles
    (150, 160, 96, 24, 4),   # 32-row decode tiles, K/32 odd
    (400, 256, 192, 32, 4),  # 128-row tiles, partly filled
    (600, 320, 384, 64, 5),  # 64-row wide tiles, three weight stages
    (264, 128, 96, 32, 4),   # 64-row prefill tiles (I/32 odd)
    (1500, 256, 192, 8, 3),  # 128-row prefill tiles
])
def test_alt_ragged(torch, T, d, I, E, k):
    wl = Workload("ragged", T=T, d=d, I=I, E=E, k=k, seed=0x5EED4000 + T + E)
    run_alt(torch, make_inputs(wl), k, 7.0, ALT, label=f"ragged{(T, d, I, E, k)}")


def test_alt_with_fast_mode(torch):
    wl = Workload("ragged", T=1500, d=256, I=192, E=8, k=3, seed=0x5EED4100)
    run_alt(torch, make_inputs(wl), 3, 7.0, ALT | moe.MOE_LAYER_MXFP6, label="alt+mxfp6")
