"""Plain fp64 CPU oracle of the attention steps beside the gpt-oss MoE layer.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

What it computes ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", section 模型架构,
Attention item; same page, "RoPE 替换了绝对位置编码" and "Attention Bias and
Attention Sinks"):
  * grouped-query attention with 64 query heads sharing 8 key/value heads;
  * layers alternate between attention limited to a band of the last 128
    positions and dense (causal) attention;
  * rotary position encoding of queries and keys;
  * each head has a learned bias logit that joins the softmax's denominator
    only, so a query may attend to no position at all.

Readings where the pages leave a step open:
  * Scores are q.k / sqrt(D), the usual scaled dot product; a head's sink is
    a logit on that same scale and carries no value.
  * Band of width W: the query at position p sees the keys at positions j
    with p - W < j <= p; dense attention sees every j <= p.
  * Query head h reads key/value head floor(h / G), G = Hq / Hkv (the query
    heads of one group are consecutive).
  * Rotary encoding rotates the pairs (x[2i], x[2i+1]) by the angle
    pos * theta^(-2i/D) with theta = 10000, the original rotary
    formulation; the pages give neither the base nor the pairing, and the
    long-context frequency rescaling they mention is not applied.
  * The head width D is not on the pages; the workloads take D = 64.

Everything is float64, from exactly the arrays the GPU receives (bf16 bit
patterns of q, k, v and fp32 sinks).
"""
from __future__ import annotations

import numpy as np

ROPE_THETA = 10000.0


def rope_angles(pos: np.ndarray, D: int, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotation angle of pair i at each position: pos * theta^(-2i/D), [n, D/2]."""
    i = np.arange(D // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / D)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(x: np.ndarray, pos: np.ndarray, theta: float = ROPE_THETA) -> np.ndarray:
    """Rotary encoding of x [n, H, D] at positions pos [n]: the pair
    (x[2i], x[2i+1]) of every head turns by rope_angles(pos)[:, i]."""
    x = np.asarray(x, dtype=np.float64)
    ang = rope_angles(pos, x.shape[-1], theta)[:, None, :]
    c, s = np.cos(ang), np.sin(ang)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * c - odd * s
    out[..., 1::2] = even * s + odd * c
    return out


def key_mask(pos: np.ndarray, S: int, window: int) -> np.ndarray:
    """Which of the key positions 0..S-1 each query position in pos [n]
    sees: [n, S] booleans."""
    p = np.asarray(pos, dtype=np.int64)[:, None]
    j = np.arange(S, dtype=np.int64)[None, :]
    ok = j <= p
    if window > 0:
        ok = ok & (j > p - window)
    return ok


def head_group(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head read by query head h."""
    return h // (Hq // Hkv)


def scores(qh: np.ndarray, kh: np.ndarray) -> np.ndarray:
    """Scaled dot products of queries [n, D] with keys [S, D]: [n, S]."""
    return qh @ kh.T / np.sqrt(qh.shape[-1])


def sink_softmax(s: np.ndarray, sink: float) -> np.ndarray:
    """Softmax of each row of s [n, S] (masked entries -inf) with the sink
    logit as one more entry of the denominator; the sink's own share is
    dropped, so a row's weights sum to less than one."""
    m = np.maximum(s.max(axis=1), float(sink))
    e = np.exp(s - m[:, None])
    return e / (e.sum(axis=1) + np.exp(float(sink) - m))[:, None]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, sinks: np.ndarray, q_pos0: int,
              window: int) -> np.ndarray:
    """q [B, Tq, Hq, D]; k, v [B, S, Hkv, D]; sinks [Hq].  Query i of a
    sequence sits at position q_pos0 + i; key j at position j."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Tq, Hq, D = q.shape
    S, Hkv = k.shape[1], k.shape[2]
    out = np.zeros((B, Tq, Hq, D))
    ok = key_mask(q_pos0 + np.arange(Tq), S, window)
    for b in range(B):
        for h in range(Hq):
            g = head_group(h, Hq, Hkv)
            w = sink_softmax(np.where(ok, scores(q[b, :, h, :], k[b, :, g, :]), -np.inf), sinks[h])
            out[b, :, h, :] = w @ v[b, :, g, :]
    return out


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, sinks: np.ndarray, q_pos0: int, window: int,
                   rows) -> np.ndarray:
    """The output rows (b, i, h) listed in rows only, one at a time (for
    sampled checks at sizes where the whole output is too slow)."""
    Hq, Hkv, S, D = q.shape[2], k.shape[2], k.shape[1], q.shape[-1]
    out = np.zeros((len(rows), D))
    for n, (b, i, h) in enumerate(rows):
        g = head_group(h, Hq, Hkv)
        ok = key_mask(np.array([q_pos0 + i]), S, window)
        qv = np.asarray(q[b, i, h], dtype=np.float64)[None, :]
        s = np.where(ok, scores(qv, np.asarray(k[b, :, g], dtype=np.float64)), -np.inf)
        out[n] = (sink_softmax(s, sinks[h]) @ np.asarray(v[b, :, g], dtype=np.float64))[0]
    return out
