"""GPU parity of the activation-quantised fast mode (moe_layer_forward_mx6):
the HIP layer through the C ABI against the fast-mode oracle (the fp64 layer
with x and h rounded to MXFP6 before the expert GEMMs) on the same seeded
inputs.  Routing must match exactly, as in the exact path; outputs within
max|err| <= 1e-2 * rms(ref) beyond the final bf16 rounding (x rounds to the
same MXFP6 values on both sides; an element of h may round the other way
where the GPU's fp32 h and the oracle's fp64 h straddle a rounding point,
which moves an output by about 1e-3 * rms).  The fast mode's deviation from
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


def run_fast(torch, inp, k, clamp, sample=None, label=""):
    E = inp["router_w"].shape[0]
    T = inp["x"].shape[0]
    say(f"fast {label} T={T} d={inp['x'].shape[1]} I={inp['w2_codes'].shape[2] * 2} E={E} k={k}")
    g = to_gpu(inp)
    out, out_f32, ids, w, counts = moe.moe_layer_forward_mx6_dbg(*[g[kk] for kk in KEYS], k=k, clamp=clamp)
    torch.cuda.synchronize()
    logits, ids_r, w_r = O.route(inp["x"], inp["router_w"], inp["router_b"], k)
    check_routing(ids.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy(),
                  dict(ids=ids_r, w=w_r, logits=logits), E)
    assert torch.equal(out, out_f32.to(torch.bfloat16))
    sel = np.arange(T) if sample is None else np.asarray(sample)
    args = (inp["x"][sel], inp["router_w"], inp["router_b"], inp, k, clamp)
    ref = O.moe_layer(*args, act="mxfp6")["y"]
    exact = O.moe_layer(*args)["y"]
    o16 = bf16_tensor_to_f64(out)[sel]
    o32 = out_f32.double().cpu().numpy()[sel]
    ex, e32 = bf16_excess(o16, ref), rel_max_err(o32, ref)
    dev = rel_max_err(o32, exact)
    say(f"fast {label}: excess/rms={ex:.3e} fp32 max/rms={e32:.3e}; deviation from the exact layer max/rms={dev:.3e}")
    assert ex <= TOL and e32 <= TOL
    # (the rounding is really applied: the exact layer is far outside the bound)
    assert dev > 10 * TOL


def test_fast_tiny(torch):
    wl = WORKLOADS["tiny"]
    run_fast(torch, make_inputs(wl), wl.k, wl.clamp, label="tiny")


def test_fast_decode_20b(torch):
    wl = WORKLOADS["20b_decode"]
    run_fast(torch, make_inputs(wl), wl.k, wl.clamp, label="20b-decode")


def test_fast_prefill_20b_sampled(torch):
    wl = WORKLOADS["20b_prefill"]
    rng = np.random.default_rng(17)
    sample = np.sort(rng.choice(wl.T, 40, replace=False))
    run_fast(torch, make_inputs(wl), wl.k, wl.clamp, sample=sample, label="20b-prefill")


@pytest.mark.parametrize("T,d,I,E,k", [
    (37, 160, 96, 24, 2),    # 16-row decode tiles, K/32 odd (byte scale copies)
    (300, 128, 128, 16, 1),  # 32-row decode tiles
    (150, 160, 96, 24, 4),   # 32-row decode tiles, K/32 odd
    (200, 96, 64, 5, 5),     # 64-row prefill tiles, K/32 odd
    (400, 256, 192, 32, 4),  # 128-row tiles, partly filled
    (600, 320, 384, 64, 5),  # 64-row wide tiles, three weight stages
    (264, 128, 96, 32, 4),   # 64-row prefill tiles (I/32 odd)
    (1500, 256, 192, 8, 3),  # 128-row prefill tiles
])
def test_fast_ragged(torch, T, d, I, E, k):
    wl = Workload("ragged", T=T, d=d, I=I, E=E, k=k, seed=0x5EED3000 + T + E)
    run_fast(torch, make_inputs(wl), k, 7.0, label=f"ragged{(T, d, I, E, k)}")
