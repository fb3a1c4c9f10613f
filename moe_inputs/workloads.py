"""Workload shapes of the gpt-oss-shaped MoE MLP layer.

Sizes follow the gpt-oss architecture summaries: 32 experts for the 20b model
and 128 for the 120b model, top-4 routing ("OpenAI 最新开源模型 gpt-oss 架构与
训练解析", 模型架构: MoE item), hidden size and expert width 2880 (same page,
gpt-oss 与 Qwen3 模型对比), 36 blocks for the 120b stack.  Each workload
carries its seed.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    I: int
    E: int
    k: int
    seed: int
    routing: str = "random"   # "random" | "zipf"
    layers: int = 1
    clamp: float = 7.0

    @property
    def pairs(self) -> int:
        return self.T * self.k


# Zipf exponent s = 1.2 for the load-imbalance workload, realised through the
# router bias b(e) = -beta * ln(rank(e)).  beta is the value for which the
# least-squares slope of log(load) against log(rank) is -1.2 on the seeded
# 120b prefill inputs (loads capped at T by construction); it was written by
# oracle/zipf_beta.py.
ZIPF_BETA = 0.559362

WORKLOADS = {
    "tiny": Workload("tiny", T=16, d=128, I=128, E=8, k=4, seed=0x5EED0000),
    "20b_decode": Workload("20b_decode", T=32, d=2880, I=2880, E=32, k=4, seed=0x5EED0001),
    "20b_prefill": Workload("20b_prefill", T=4096, d=2880, I=2880, E=32, k=4, seed=0x5EED0002),
    # a mid-sized batch (32 rows per expert on average: the largest batch
    # the decode kernels take)
    "20b_batch256": Workload("20b_batch256", T=256, d=2880, I=2880, E=32, k=4, seed=0x5EED0006),
    "120b_prefill_zipf": Workload("120b_prefill_zipf", T=8192, d=2880, I=2880, E=128, k=4,
                                  seed=0x5EED0003, routing="zipf"),
    "120b_stack36": Workload("120b_stack36", T=2048, d=2880, I=2880, E=128, k=4,
                             seed=0x5EED1000, layers=36),
    # The contrast model of the same page's gpt-oss / Qwen3 comparison
    # ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", gpt-oss 与 Qwen3 模型对比):
    # width 2048, expert projection 768, 128 experts with 8 active per token.
    "qwen3_decode": Workload("qwen3_decode", T=32, d=2048, I=768, E=128, k=8, seed=0x5EED0004),
    "qwen3_prefill": Workload("qwen3_prefill", T=4096, d=2048, I=768, E=128, k=8, seed=0x5EED0005),
}


@dataclass(frozen=True)
class AttnWorkload:
    """One call of the attention steps: B sequences, each with Tq queries at
    positions q_pos0 .. q_pos0 + Tq - 1 over S cached keys at positions
    0 .. S - 1; window 0 is dense (causal) attention, otherwise the band of
    the last `window` positions."""
    name: str
    B: int
    Tq: int
    S: int
    q_pos0: int
    Hq: int
    Hkv: int
    D: int
    window: int
    seed: int


# 64 query heads over 8 key/value heads, layers alternating between a
# 128-position band and dense attention ("OpenAI 最新开源模型 gpt-oss 架构与训练
# 解析", 模型架构: Attention item); head width 64 (not on the pages).  The
# prefill cases are one 4096-token sequence, the decode cases one new token
# for each of 32 sequences with 4096 cached positions, and the chunk cases
# the last 256 tokens of a 4096-token sequence.
ATTN_WORKLOADS = {
    "attn_tiny_band": AttnWorkload("attn_tiny_band", B=2, Tq=40, S=40, q_pos0=0, Hq=16, Hkv=2, D=64, window=16,
                                   seed=0x5EED2000),
    "attn_tiny_dense": AttnWorkload("attn_tiny_dense", B=2, Tq=40, S=40, q_pos0=0, Hq=16, Hkv=2, D=64, window=0,
                                    seed=0x5EED2001),
    "attn_prefill_band": AttnWorkload("attn_prefill_band", B=1, Tq=4096, S=4096, q_pos0=0, Hq=64, Hkv=8, D=64,
                                      window=128, seed=0x5EED2002),
    "attn_prefill_dense": AttnWorkload("attn_prefill_dense", B=1, Tq=4096, S=4096, q_pos0=0, Hq=64, Hkv=8, D=64,
                                       window=0, seed=0x5EED2003),
    "attn_decode_band": AttnWorkload("attn_decode_band", B=32, Tq=1, S=4096, q_pos0=4095, Hq=64, Hkv=8, D=64,
                                     window=128, seed=0x5EED2004),
    "attn_decode_dense": AttnWorkload("attn_decode_dense", B=32, Tq=1, S=4096, q_pos0=4095, Hq=64, Hkv=8, D=64,
                                      window=0, seed=0x5EED2005),
    "attn_chunk_dense": AttnWorkload("attn_chunk_dense", B=2, Tq=256, S=4096, q_pos0=3840, Hq=64, Hkv=8, D=64,
                                     window=0, seed=0x5EED2006),
    "attn_chunk_band": AttnWorkload("attn_chunk_band", B=2, Tq=256, S=4096, q_pos0=3840, Hq=64, Hkv=8, D=64,
                                    window=128, seed=0x5EED2007),
}
