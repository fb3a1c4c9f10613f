"""GPU parity of the attention steps beside the MoE layer (rotary encoding,
grouped-query attention with a 128-position band or dense causal masking and
per-head sink logits; "OpenAI 最新开源模型 gpt-oss 架构与训练解析", 模型架构:
Attention item) against the fp64 oracle, through the C ABI.

Tolerances:
* attention: max over elements of (|out - ref| - half a bf16 ulp of ref)
  <= ATT_TOL * rms(ref).  The kernel's own error is far below the final
  bf16 rounding: scores are sums of 64 exact bf16 products in fp32, the
  softmax is fp32 (hardware exp2, about 1 ulp), the probabilities enter the
  value products as two bf16 terms (relative error about 2^-17), and the
  output sums run in fp32 over at most a few thousand keys (about 1e-5
  relative); the bound keeps an order of magnitude above that.
* rotary encoding: the same measure against the exact rotation of the bf16
  input, bounded by 1e-5 * rms(x) (the rotation is fp32 before the single
  rounding to bf16).
* rotary encoding followed by attention: the rotary entry point stores
  bf16, so the oracle rounds its exact rotation to bf16 before attending.
  Where the kernel's fp32 rotation and the exact one sit on either side of
  a rounding boundary, one element differs by one bf16 ulp; that moves a
  score by about 2^-8 |q_i k_i| / sqrt(D), about 1e-3, and the output by
  about that relative amount.  Bounded by 5e-3 * rms(ref).  (Against the
  unrounded rotation the bf16 storage of q and k alone moves the output by
  up to 3e-2 of its rms on this case.)
"""
import sys

import numpy as np
import pytest

from moe_inputs import synth
from moe_inputs.workloads import ATTN_WORKLOADS
from oracle import attention_oracle as A
from oracle.moe_oracle import bf16_bits_to_f64, round_to_bf16
import sparse_moe_transformer_softmax_amd as moe

pytestmark = pytest.mark.gpu

ATT_TOL = 1e-4
ROPE_TOL = 1e-5
E2E_TOL = 5e-3


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "no GPU"
    moe.lib()
    return _t


def _dev(torch, bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")


def _host(t):
    import torch
    return bf16_bits_to_f64(t.detach().cpu().view(torch.int16).numpy().view(np.uint16))


def _excess(out, ref):
    """max(|out - ref| - half an ulp of ref) / rms(ref), and the raw max/rms."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    _, e = np.frexp(ref)
    half_ulp = np.ldexp(1.0, e - 9)
    err = np.abs(out - ref)
    return float(np.max(err - half_ulp)) / rms, float(np.max(err)) / rms


def _run(torch, q, k, v, sinks, q_pos0, window):
    out = moe.moe_attn_forward(_dev(torch, q), _dev(torch, k), _dev(torch, v),
                               torch.from_numpy(sinks).to("cuda:0"), q_pos0=q_pos0, window=window)
    torch.cuda.synchronize()
    return _host(out)


def _inputs(B, Tq, S, Hq, Hkv, seed):
    return synth.gen_attention(seed, B, Tq, S, Hq, Hkv, 64)


SMALL = [
    # B, Tq, S, q_pos0, Hq, Hkv, window
    (2, 40, 40, 0, 16, 2, 16),     # ragged query blocks and a partial key tile
    (2, 40, 40, 0, 16, 2, 0),
    (1, 1, 1, 0, 8, 1, 0),         # one key
    (1, 70, 70, 0, 4, 4, 1),       # a band of one: each query sees itself only
    (1, 50, 50, 0, 4, 2, 100),     # band wider than the sequence
    (3, 33, 97, 64, 16, 1, 0),     # sixteen heads per group, a chunk at position 64
    (2, 5, 300, 295, 8, 2, 128),   # a few queries at the end of a long cache (key split)
    (2, 1, 257, 256, 64, 8, 0),    # decode, the key split
    (2, 1, 257, 256, 64, 8, 128),
    (1, 64, 64, 0, 2, 1, 24),      # two heads per group
]


@pytest.mark.parametrize("B,Tq,S,q_pos0,Hq,Hkv,window", SMALL)
def test_attention_small_shapes(torch, B, Tq, S, q_pos0, Hq, Hkv, window):
    say(f"attn small B={B} Tq={Tq} S={S} q_pos0={q_pos0} Hq={Hq} Hkv={Hkv} window={window}")
    q, k, v, sinks = _inputs(B, Tq, S, Hq, Hkv, seed=1000 + Tq + S + window)
    out = _run(torch, q, k, v, sinks, q_pos0, window)
    ref = A.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), sinks.astype(np.float64),
                      q_pos0, window)
    ex, raw = _excess(out, ref)
    say(f"  excess/rms={ex:.3e} raw/rms={raw:.3e}")
    assert ex <= ATT_TOL


def test_attention_without_sinks(torch):
    say("attn sinks -inf")
    q, k, v, _ = _inputs(2, 40, 40, 16, 2, seed=77)
    sinks = np.full(16, -np.inf, dtype=np.float32)
    out = _run(torch, q, k, v, sinks, 0, 8)
    ref = A.attention(bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v), sinks.astype(np.float64), 0, 8)
    ex, raw = _excess(out, ref)
    say(f"  excess/rms={ex:.3e}")
    assert np.isfinite(out).all() and ex <= ATT_TOL


@pytest.mark.parametrize("name", sorted(ATTN_WORKLOADS))
def test_attention_workloads(torch, name):
    wl = ATTN_WORKLOADS[name]
    say(f"attn workload {name}")
    q, k, v, sinks = synth.gen_attention(wl.seed, wl.B, wl.Tq, wl.S, wl.Hq, wl.Hkv, wl.D)
    out = _run(torch, q, k, v, sinks, wl.q_pos0, wl.window)
    qf, kf, vf = bf16_bits_to_f64(q), bf16_bits_to_f64(k), bf16_bits_to_f64(v)
    if wl.B * wl.Tq * wl.Hq * wl.S <= 140_000_000:
        ref = A.attention(qf, kf, vf, sinks.astype(np.float64), wl.q_pos0, wl.window)
        ex, raw = _excess(out, ref)
        say(f"  all rows: excess/rms={ex:.3e} raw/rms={raw:.3e}")
    else:
        # sampled rows: the first and last positions, the band and tile edges,
        # and random ones, over all heads of two groups
        rng = np.random.default_rng(wl.seed)
        idx = sorted(set([0, 1, 31, 32, 33, 127, 128, 129, wl.Tq - 1] + list(rng.integers(0, wl.Tq, 24))))
        idx = [i for i in idx if i < wl.Tq]
        heads = sorted(set(list(range(wl.Hq // wl.Hkv)) + list(rng.integers(0, wl.Hq, 6))))
        rows = [(int(rng.integers(0, wl.B)), i, h) for i in idx for h in heads]
        ref = A.attention_rows(qf, kf, vf, sinks.astype(np.float64), wl.q_pos0, wl.window, rows)
        got = np.stack([out[b, i, h] for b, i, h in rows])
        rms_all = float(np.sqrt(np.mean(out ** 2)))
        ex, raw = _excess(got, ref)
        say(f"  {len(rows)} sampled rows: excess/rms={ex:.3e} raw/rms={raw:.3e} (rms of all rows {rms_all:.3e})")
        assert np.isfinite(out).all()
    assert ex <= ATT_TOL


def test_attention_is_deterministic(torch):
    wl = ATTN_WORKLOADS["attn_decode_dense"]
    say("attn determinism (decode, key split)")
    q, k, v, sinks = synth.gen_attention(wl.seed, wl.B, wl.Tq, wl.S, wl.Hq, wl.Hkv, wl.D)
    a = _run(torch, q, k, v, sinks, wl.q_pos0, wl.window)
    b = _run(torch, q, k, v, sinks, wl.q_pos0, wl.window)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("n,H,pos0", [(40, 16, 0), (7, 8, 4089), (33, 2, 131000), (1, 64, 0)])
def test_rope(torch, n, H, pos0):
    say(f"rope n={n} H={H} pos0={pos0}")
    x = synth.f32_to_bf16_bits(np.random.default_rng(n + H).standard_normal((n, H, 64), dtype=np.float32))
    xd = _dev(torch, x)
    out = _host(moe.moe_attn_rope(xd, pos0=pos0))
    torch.cuda.synchronize()
    xf = bf16_bits_to_f64(x)
    ref = A.rope(xf, pos0 + np.arange(n))
    rms_x = float(np.sqrt(np.mean(xf ** 2)))
    _, e = np.frexp(ref)
    ex = float(np.max(np.abs(out - ref) - np.ldexp(1.0, e - 9))) / rms_x
    say(f"  excess/rms(x)={ex:.3e}")
    assert ex <= ROPE_TOL
    # in place gives the same bits
    moe.moe_attn_rope(xd, pos0=pos0, out=xd)
    torch.cuda.synchronize()
    assert np.array_equal(_host(xd), out)


def test_rope_then_attention(torch):
    say("rope + attention end to end")
    B, T, Hq, Hkv = 1, 300, 16, 2
    q, k, v, sinks = _inputs(B, T, T, Hq, Hkv, seed=4242)
    qd, kd = _dev(torch, q), _dev(torch, k)
    qr = moe.moe_attn_rope(qd.view(T, Hq, 64)).view(B, T, Hq, 64)
    kr = moe.moe_attn_rope(kd.view(T, Hkv, 64)).view(B, T, Hkv, 64)
    out = moe.moe_attn_forward(qr, kr, _dev(torch, v), torch.from_numpy(sinks).to("cuda:0"), window=128)
    torch.cuda.synchronize()
    pos = np.arange(T)
    qo = round_to_bf16(A.rope(bf16_bits_to_f64(q)[0], pos))[None]
    ko = round_to_bf16(A.rope(bf16_bits_to_f64(k)[0], pos))[None]
    ref = A.attention(qo, ko, bf16_bits_to_f64(v), sinks.astype(np.float64), 0, 128)
    ex, raw = _excess(_host(out), ref)
    say(f"  excess/rms={ex:.3e} raw/rms={raw:.3e}")
    assert ex <= E2E_TOL
