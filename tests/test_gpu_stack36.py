"""The 36-layer stack of gpt-oss-120b-shaped MoE layers (T 2048, E 128,
d = I = 2880, top-4, RMSNorm with eps 1e-5 and a residual add between
layers; "OpenAI 最新开源模型 gpt-oss 架构与训练解析", RMSNorm 替换 LayerNorm)
at its full depth on one GPU, checked two ways:

* every one of the 36 seeded layers against the fp64 oracle on its own
  gap-conditioned input: expert ids and per-expert counts bit-exact and gate
  weights to 4e-6 on all 2048 tokens, and the layer output on two sampled
  tokens within the bf16 bound;
* the stack entry point against its own steps -- RMSNorm, the layer, the
  fused residual add + RMSNorm -- called layer by layer through the C ABI,
  bit for bit, over all 36 layers.

The oracle takes no input from the GPU path, so the stack's later layers,
whose inputs come out of the computation, are covered by the composition
check and by each layer's own seeded check rather than by teacher forcing.
All 36 layers' weights (61 GB) stay resident on the GPU.
"""
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from oracle.workload_inputs import make_inputs
from moe_inputs.workloads import WORKLOADS
import sparse_moe_transformer_softmax_amd as moe
from tests.parity_util import KEYS, TOL, bf16_excess, bf16_tensor_to_f64, check_routing, rel_max_err, to_gpu

pytestmark = pytest.mark.gpu

LAYER_KEYS = ["router_w", "router_b", "w13_codes", "w13_scales", "b13", "w2_codes", "w2_scales", "b2"]


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "no GPU"
    moe.lib()
    return _t


@pytest.mark.timeout(900)
def test_stack36_every_layer_and_the_composition(torch):
    wl = WORKLOADS["120b_stack36"]
    rng = np.random.default_rng(36)
    layers, x0 = [], None
    worst = 0.0
    for l in range(wl.layers):
        inp = make_inputs(wl, layer=l)
        if l == 0:
            x0 = inp["x"]
        g = to_gpu(inp)
        out, out_f32, ids, w, counts = moe.moe_layer_forward_dbg(*[g[kk] for kk in KEYS], k=wl.k, clamp=wl.clamp)
        torch.cuda.synchronize()
        logits, ids_r, w_r = O.route(inp["x"], inp["router_w"], inp["router_b"], wl.k)
        check_routing(ids.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy(),
                      dict(ids=ids_r, w=w_r, logits=logits), wl.E)
        assert torch.equal(out, out_f32.to(torch.bfloat16))
        sel = np.sort(rng.choice(wl.T, 2, replace=False))
        ref = O.moe_layer(inp["x"][sel], inp["router_w"], inp["router_b"], inp, wl.k, wl.clamp)["y"]
        ex = bf16_excess(bf16_tensor_to_f64(out)[sel], ref)
        e32 = rel_max_err(out_f32.double().cpu().numpy()[sel], ref)
        worst = max(worst, ex, e32)
        say(f"stack36 layer {l}: routing exact on {wl.T} tokens (counts max {int(counts.max())}), "
            f"tokens {sel.tolist()} excess/rms={ex:.2e} fp32 max/rms={e32:.2e}")
        assert ex <= TOL and e32 <= TOL
        layers.append({kk: g[kk] for kk in LAYER_KEYS})
        del g, inp, out, out_f32
    say(f"stack36: all layers within the bound (worst {worst:.2e})")

    x = torch.from_numpy(np.ascontiguousarray(x0).view(np.int16)).view(torch.bfloat16).cuda()
    got = moe.moe_stack_forward(x, layers, k=wl.k, clamp=wl.clamp, eps=1e-5)
    n = moe.moe_rmsnorm(x, 1e-5)
    for l, L in enumerate(layers):
        _, out_f32, _, _, _ = moe.moe_layer_forward_dbg(n, *[L[kk] for kk in LAYER_KEYS], k=wl.k, clamp=wl.clamp)
        x, n = moe.moe_rmsnorm_residual(x, out_f32, 1e-5)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(got.float()).all())
    assert torch.equal(got, x)
    say("stack36: the stack equals its steps bit for bit over 36 layers")
