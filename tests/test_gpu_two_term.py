"""GPU parity of the two-term activation option (MOE_LAYER_MX6X2 of
moe_layer_forward_ex): the HIP layer through the C ABI against the oracle's
two-term layer (the fp64 layer with x and h rounded to two MXFP6 terms
before the expert GEMMs, mx6x2_quantize) on the same seeded inputs.
Routing must match exactly; outputs within max|err| <= 1e-2 * rms(ref)
beyond the final bf16 rounding, as for the exact path.  x rounds to the
same two terms on both sides (the residual of a bf16 value after its first
term is exact in fp32); an element of h can round differently only where
the GPU's fp32 h and the oracle's fp64 h straddle a rounding point of a
term, which is rare and moves an output by far less than the bound.  That
the two-term arithmetic is what runs is checked by the output lying much
closer to the two-term oracle than to the exact layer; the deviation from
the exact layer is printed."""
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


def run_two(torch, inp, k, clamp, sample=None, label="", alt=False):
    E = inp["router_w"].shape[0]
    T = inp["x"].shape[0]
    say(f"two-term {label} T={T} d={inp['x'].shape[1]} I={inp['w2_codes'].shape[2] * 2} E={E} k={k} alt={alt}")
    g = to_gpu(inp)
    flags = moe.MOE_LAYER_MX6X2 | (moe.MOE_LAYER_ALT_ACT if alt else 0)
    out, out_f32, ids, w, counts = moe.moe_layer_forward_ex(*[g[kk] for kk in KEYS], k=k, clamp=clamp, flags=flags,
                                                            debug=True)
    torch.cuda.synchronize()
    logits, ids_r, w_r = O.route(inp["x"], inp["router_w"], inp["router_b"], k)
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy(),
                  dict(ids=ids_r, w=w_r, logits=logits), E)
    assert torch.equal(out, out_f32.to(torch.bfloat16))
    sel = np.arange(T) if sample is None else np.asarray(sample)
    args = (inp["x"][sel], inp["router_w"], inp["router_b"], inp, k, clamp)
    ref = O.moe_layer(*args, act="mx6x2", alt=alt)["y"]
    exact = O.moe_layer(*args, alt=alt)["y"]
    o16 = bf16_tensor_to_f64(out)[sel]
    o32 = out_f32.double().cpu().numpy()[sel]
    ex, e32 = bf16_excess(o16, ref), rel_max_err(o32, ref)
    dev = rel_max_err(o32, exact)
    say(f"two-term {label}: excess/rms={ex:.3e} fp32 max/rms={e32:.3e}; "
        f"deviation from the exact layer max/rms={dev:.3e}")
    assert ex <= TOL and e32 <= TOL
    assert e32 < dev / 5, (e32, dev)
    return out


def test_two_term_tiny(torch):
    wl = WORKLOADS["tiny"]
    run_two(torch, make_inputs(wl), wl.k, wl.clamp, label="tiny")


def test_two_term_decode_20b(torch):
    wl = WORKLOADS["20b_decode"]
    run_two(torch, make_inputs(wl), wl.k, wl.clamp, label="20b-decode")


def test_two_term_prefill_20b_sampled(torch):
    wl = WORKLOADS["20b_prefill"]
    rng = np.random.default_rng(23)
    sample = np.sort(rng.choice(wl.T, 40, replace=False))
    run_two(torch, make_inputs(wl), wl.k, wl.clamp, sample=sample, label="20b-prefill")


@pytest.mark.parametrize("T,d,I,E,k", [
    (37, 160, 96, 24, 2),    # 16-row decode tiles, K/32 odd (byte scale copies)
    (300, 128, 128, 16, 1),  # 32-row decode tiles
    (150, 160, 96, 24, 4),   # 32-row decode tiles, K/32 odd
    (200, 96, 64, 5, 5),     # 64-row prefill tiles, K/32 odd
    (400, 256, 192, 32, 4),  # 128-row tiles, partly filled
    (600, 320, 384, 64, 5),  # 64-row wide tiles, three weight stages
    (264, 128, 96, 32, 4),   # 64-row prefill tiles (I/32 odd)
    (1500, 256, 192, 8, 3),  # 128-row prefill tiles
    (8, 4160, 64, 8, 4),     # decode, K above 4096 (the phase loop)
])
def test_two_term_ragged(torch, T, d, I, E, k):
    wl = Workload("ragged", T=T, d=d, I=I, E=E, k=k, seed=0x5EED3500 + T + E)
    run_two(torch, make_inputs(wl), k, 7.0, label=f"ragged{(T, d, I, E, k)}")


def test_two_term_with_variant_activation(torch):
    wl = Workload("ragged", T=1500, d=256, I=192, E=8, k=3, seed=0x5EED3600)
    sample = np.sort(np.random.default_rng(3).choice(wl.T, 48, replace=False))
    run_two(torch, make_inputs(wl), wl.k, 7.0, sample=sample, label="alt", alt=True)


@pytest.mark.parametrize("name", ["20b_decode", "20b_prefill"])
def test_two_term_packed_equals_row_major_bitwise(torch, name):
    wl = WORKLOADS[name]
    say(f"two-term packed vs row-major {name}")
    g = to_gpu(make_inputs(wl, condition=False))
    p = dict(g)
    p["w13_codes"], p["w13_scales"] = moe.moe_pack_weights(g["w13_codes"], g["w13_scales"])
    p["w2_codes"], p["w2_scales"] = moe.moe_pack_weights(g["w2_codes"], g["w2_scales"])
    a = moe.moe_layer_forward_ex(*[g[k] for k in KEYS], k=wl.k, clamp=wl.clamp, flags=moe.MOE_LAYER_MX6X2,
                                 debug=True)
    b = moe.moe_layer_forward_ex(*[p[k] for k in KEYS], k=wl.k, clamp=wl.clamp,
                                 flags=moe.MOE_LAYER_MX6X2 | moe.MOE_LAYER_PACKED, debug=True)
    torch.cuda.synchronize()
    for x, y, what in zip(a, b, ["out", "out_f32", "ids", "w", "counts"]):
        assert torch.equal(x, y), what
