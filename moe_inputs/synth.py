"""Seeded synthetic inputs for the gpt-oss-shaped MoE MLP layer.

This module draws random numbers and encodes them into the storage formats
the layer consumes (bf16 activations, bf16 router weight, fp32 biases,
MXFP4 expert weights as raw E2M1 nibbles plus E8M0 scale bytes).  It holds
none of the layer's arithmetic: no matrix product, no routing, no
activation.  Both the GPU path and the CPU oracle read its output.

Generator: numpy's Philox-4x64 counter-based generator (Salmon et al.,
"Parallel random numbers: as easy as 1, 2, 3", SC'11), keyed by
(seed, stream id).  Every tensor has its own stream id, so tensors can be
drawn in any order or in part.

Distributions (workload description of the layer, see the gpt-oss
architecture summaries, "模型架构 / MoE" and "权重量化" entries):
  x       ~ N(0, 1), rounded to bf16 (round to nearest even)
  W_r     ~ N(0, 1/d), rounded to bf16
  b_r     ~ N(0, 0.1)  (second argument is the variance)
  codes   uniform over all 16 E2M1 nibbles
  scales  E8M0 bytes uniform in {121, 122, 123, 124} (2^-6 .. 2^-3)
  b13, b2 ~ N(0, 0.01)

Attention inputs (the attention steps next to the layer; "OpenAI 最新开源模型
gpt-oss 架构与训练解析", 模型架构: Attention item):
  q, k, v ~ N(0, 1), rounded to bf16, layouts [B, T, H, D]
  sinks   uniform in [-2, 6] (one logit per query head; wide enough that the
          sink ranges from negligible to dominant against a 128-key band)
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream ids, one per tensor kind
_S_X, _S_X_REDRAW, _S_WR, _S_BR, _S_W13C, _S_W13S, _S_B13, _S_W2C, _S_W2S, _S_B2, _S_PERM = range(11)
_S_AQ, _S_AK, _S_AV, _S_ASINK = range(11, 15)

SCALE_LO = 121  # E8M0 byte for 2^-6
SCALE_HI = 124  # E8M0 byte for 2^-3


def _gen(seed: int, stream: int, *extra: int) -> np.random.Generator:
    key = [int(seed) & 0xFFFFFFFFFFFFFFFF, (int(stream) << 48) ^ (len(extra) << 40)]
    ctr = [0, 0, 0, 0]
    for i, v in enumerate(extra[:2]):
        ctr[2 + i] = int(v) & 0xFFFFFFFFFFFFFFFF
    return np.random.Generator(np.random.Philox(key=key, counter=ctr))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode float32 values as bf16 bit patterns (uint16), round to nearest even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u >> 16) & 1) + 0x7FFF
    out = ((u + r) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


# Bulk byte draws are split into chunks of CHUNK_WORDS 64-bit words; chunk c
# of a stream comes from its own Philox counter block (the chunk index is
# the third counter word), so the chunks can be drawn in parallel threads
# (numpy's bit generators release the interpreter lock while they fill).
CHUNK_WORDS = 1 << 21


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _random_bytes(seed: int, stream: int, n: int) -> np.ndarray:
    """n uniformly random bytes of (seed, stream), chunk by chunk."""
    words = (n + 7) // 8
    buf = np.empty(words, dtype=np.uint64)
    nchunk = (words + CHUNK_WORDS - 1) // CHUNK_WORDS

    def fill(c: int) -> None:
        lo = c * CHUNK_WORDS
        hi = min(words, lo + CHUNK_WORDS)
        buf[lo:hi] = _gen(seed, stream, c).bit_generator.random_raw(hi - lo)

    if nchunk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(min(_threads(), nchunk)) as ex:
            list(ex.map(fill, range(nchunk)))
    return buf.view(np.uint8)[:n]


def gen_x(seed: int, T: int, d: int, redraw: dict[int, int] | None = None) -> np.ndarray:
    """Activations, bf16 bits [T, d].  ``redraw`` maps a row to a redraw
    attempt number; such rows come from a separate counter block."""
    g = _gen(seed, _S_X)
    x = f32_to_bf16_bits(g.standard_normal((T, d), dtype=np.float32))
    if redraw:
        for row, attempt in redraw.items():
            gr = _gen(seed, _S_X_REDRAW, row, attempt)
            x[row] = f32_to_bf16_bits(gr.standard_normal(d, dtype=np.float32))
    return x


def gen_router(seed: int, E: int, d: int, bias_std: float = float(np.sqrt(0.1))):
    """Router weight bf16 bits [E, d] ~ N(0, 1/d) and bias fp32 [E] ~ N(0, 0.1)."""
    w = _gen(seed, _S_WR).standard_normal((E, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    b = (_gen(seed, _S_BR).standard_normal(E) * bias_std).astype(np.float32)
    return f32_to_bf16_bits(w), b


def zipf_router_bias(seed: int, E: int, beta: float) -> np.ndarray:
    """Router bias b(e) = -beta * ln(rank(e)), rank a seeded permutation of 1..E."""
    rank = _gen(seed, _S_PERM).permutation(E) + 1
    return (-beta * np.log(rank.astype(np.float64))).astype(np.float32)


def gen_mxfp4(seed: int, stream_codes: int, stream_scales: int, E: int, rows: int, K: int):
    """MXFP4 matrix stack: codes uint8 [E, rows, K/2], scales uint8 [E, rows, K/32]."""
    assert K % 32 == 0
    codes = _random_bytes(seed, stream_codes, E * rows * (K // 2)).reshape(E, rows, K // 2)
    sb = _random_bytes(seed, stream_scales, E * rows * (K // 32)).reshape(E, rows, K // 32)
    scales = (sb & np.uint8(3)) + np.uint8(SCALE_LO)
    return codes, scales


def gen_experts(seed: int, E: int, d: int, I: int):
    """Expert weights: dict with w13_codes [E,2I,d/2], w13_scales [E,2I,d/32],
    b13 fp32 [E,2I], w2_codes [E,d,I/2], w2_scales [E,d,I/32], b2 fp32 [E,d]."""
    w13c, w13s = gen_mxfp4(seed, _S_W13C, _S_W13S, E, 2 * I, d)
    w2c, w2s = gen_mxfp4(seed, _S_W2C, _S_W2S, E, d, I)
    b13 = (_gen(seed, _S_B13).standard_normal((E, 2 * I)) * 0.1).astype(np.float32)
    b2 = (_gen(seed, _S_B2).standard_normal((E, d)) * 0.1).astype(np.float32)
    return dict(w13_codes=w13c, w13_scales=w13s, b13=b13, w2_codes=w2c, w2_scales=w2s, b2=b2)


def gen_attention(seed: int, B: int, Tq: int, S: int, Hq: int, Hkv: int, D: int):
    """q bf16 bits [B, Tq, Hq, D], k and v bf16 bits [B, S, Hkv, D], sinks fp32 [Hq]."""
    q = f32_to_bf16_bits(_gen(seed, _S_AQ).standard_normal((B, Tq, Hq, D), dtype=np.float32))
    k = f32_to_bf16_bits(_gen(seed, _S_AK).standard_normal((B, S, Hkv, D), dtype=np.float32))
    v = f32_to_bf16_bits(_gen(seed, _S_AV).standard_normal((B, S, Hkv, D), dtype=np.float32))
    sinks = _gen(seed, _S_ASINK).uniform(-2.0, 6.0, Hq).astype(np.float32)
    return q, k, v, sinks
