"""Bitwise one-hot probe of the expert GEMMs' operand layouts.

Each token is a one-hot row x = e_j (bf16 1.0 at column j) and is routed to
one expert (k = 1, so its gate weight is exactly 1).  Every expert e keeps
one intermediate column i*(e) alive: its gate row has bias 64 and scale
2^-3 (so g = 64 + W_gate[i*, j] lies in [63.25, 64.75], where the sigmoid is
1 to within 2^-90 in both fp32 and fp64), all other gate rows have bias
-1024 (h = 0 there), and its up row holds only codes whose value plus one is
a power of two (0, -0.5, 1, 3 at scale 1).  With no clamp, h is zero except

    h[i*] = (64 + W_gate[e, i*, j]) * (1 + W_up[e, i*, j])

and the layer output is out[t, r] = W2[e, r, i*] * h[i*]: one nonzero product
per element at every step.  h[i*] needs at most two FP6 terms and every
product and partial sum is exact in fp32, so the GPU's fp32 output must equal
the fp32 rounding of the fp64 oracle bit for bit.  A swapped nibble, a scale
byte taken from the wrong block, a gate/up mix-up, a transposed operand or a
lane mapped to the wrong row or K position moves a value and fails the
comparison.  (The expert weights of the MXFP4 format: "OpenAI 最新开源模型
gpt-oss 架构与训练解析", 权重量化 item.)
"""
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from moe_inputs import synth
import sparse_moe_transformer_softmax_amd as moe
from tests.parity_util import KEYS, to_gpu

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


UP_CODES = np.array([0, 9, 2, 5], dtype=np.uint8)  # E2M1 values 0, -0.5, 1, 3: value + 1 a power of two


def probe_inputs(T, d, I, E, alt, seed):
    rng = np.random.default_rng(seed)
    ex = synth.gen_experts(seed, E, d, I)
    w13c, w13s = ex["w13_codes"].copy(), ex["w13_scales"].copy()
    b13 = np.zeros((E, 2 * I), dtype=np.float32)
    istar = rng.choice(I, E, replace=E > I)
    cols = np.arange(I)
    gate_rows = 2 * cols if alt else cols
    up_rows = 2 * cols + 1 if alt else I + cols
    for e in range(E):
        b13[e, gate_rows] = -1024.0
        b13[e, up_rows] = 0.0
        gr, ur = gate_rows[istar[e]], up_rows[istar[e]]
        b13[e, gr] = 64.0
        w13s[e, gr, :] = 124
        w13s[e, ur, :] = 127
        up = UP_CODES[rng.integers(0, 4, d)]
        w13c[e, ur, :] = up[0::2] | (up[1::2] << 4)
    # router: column j sends its token to expert route_col[j] with a logit
    # gap of 1
    route_col = rng.integers(0, E, d)
    wr = np.zeros((E, d), dtype=np.float32)
    wr[route_col, np.arange(d)] = 1.0
    j = rng.integers(0, d, T)
    x = np.zeros((T, d), dtype=np.uint16)
    x[np.arange(T), j] = 0x3F80
    return dict(x=x, router_w=synth.f32_to_bf16_bits(wr), router_b=np.zeros(E, dtype=np.float32),
                w13_codes=w13c, w13_scales=w13s, b13=b13, w2_codes=ex["w2_codes"], w2_scales=ex["w2_scales"],
                b2=np.zeros((E, d), dtype=np.float32)), route_col[j]


# (T, d, I, E): 16-row decode tiles with the folded combine; 32-row decode
# tiles; 64-row prefill tiles (K/32 odd); 128-row prefill tiles
CASES = [(64, 256, 128, 16), (200, 256, 128, 8), (600, 288, 96, 8), (600, 256, 128, 8)]


@pytest.mark.parametrize("alt", [False, True], ids=["gate-first", "interleaved"])
@pytest.mark.parametrize("T,d,I,E", CASES)
def test_one_hot_probe_is_bit_exact(torch, T, d, I, E, alt):
    inp, experts = probe_inputs(T, d, I, E, alt, seed=0x5EED4000 + T + d + I + E + alt)
    say(f"one-hot probe T={T} d={d} I={I} E={E} alt={alt}")
    g = to_gpu(inp)
    flags = moe.MOE_LAYER_ALT_ACT if alt else 0
    out, out_f32, ids, w, counts = moe.moe_layer_forward_ex(*[g[kk] for kk in KEYS], k=1, clamp=float("inf"),
                                                            flags=flags, debug=True)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy()[:, 0], experts)
    assert np.all(w.cpu().numpy() == 1.0)
    with np.errstate(over="ignore"):
        ref = O.moe_layer(inp["x"], inp["router_w"], inp["router_b"], inp, 1, np.inf, alt=alt)["y"]
    want = ref.astype(np.float32)
    got = out_f32.cpu().numpy()
    assert np.count_nonzero(want) > want.size // 2  # the probe carries values
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:4].tolist()}"
    assert torch.equal(out, out_f32.to(torch.bfloat16))
