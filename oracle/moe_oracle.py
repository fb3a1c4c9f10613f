"""Plain fp64 CPU oracle of the gpt-oss mixture-of-experts MLP layer.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it and shares no code with it.

Everything is computed in float64 from exactly the arrays the GPU receives
(bf16 bit patterns, fp32 biases, raw MXFP4 nibbles and E8M0 scale bytes).

Sources (web pages on gpt-oss; cited by page title and section):
  [A] "OpenAI 最新开源模型 gpt-oss 架构与训练解析" (dtcms.com/a/486625):
      section 模型架构, MoE item (top-4 routing, softmax weighting of the
      selected experts, gated-SwiGLU FFN with clamp and residual);
      权重量化 item (MoE weights in MXFP4, 4.25 bits per weight);
      Swish/SwiGLU 替换 GELU (Swish(x) = x * sigmoid(x));
      RMSNorm 替换 LayerNorm (divide by the root mean square, no bias).
  [B] "【LLM】GPT-OSS架构变化详解" (dtcms.com/a/386406.html):
      2.4.1 MoE 的核心原理 (a router scores the experts of each token;
      the unselected experts do nothing for that token).
  [C] Xin Zhiyuan's translation of Raschka's "From GPT-2 to gpt-oss"
      (dreamgost.com/a/xinwen/gongsixinwen/564.html): the GLU variant has
      three linear layers (gate, up, and the down projection).

Readings where the pages leave a step open (each one is plain and is the one
the rest of the pages support):
  * MXFP4 = OCP microscaling FP4: E2M1 element codes, one E8M0 scale byte
    per 32 consecutive elements of a row, scale 2^(s-127), byte 0xFF = NaN;
    two codes per byte, the low nibble holds the even element.
  * Top-k ties go to the lower expert index; slots are ordered by
    descending logit.
  * The softmax runs over the k selected logits only.
  * The clamp limit c applies symmetrically to gate and up, before the
    sigmoid and before the +1; h = clamp(g) * sigmoid(clamp(g)) * (clamp(u) + 1).
  * The fused gate/up weight holds the gate rows first ([0, I)) and the up
    rows second ([I, 2I)); both expert biases live inside the expert, so the
    down bias is weighted by the gate weight of its slot.
  * RMSNorm uses eps = 1e-5 and unit gain; in the layer stack the residual
    stream and each layer's normalised input are stored as bf16.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  bf16 is the upper half of an
    IEEE binary32, so the value is exact in float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), returned as float64.
    Exact for normal results (8 significant bits); NaN/inf pass through."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)   # np.rint: half to even
    return np.where(np.isfinite(v), r, v)


def e2m1_value(code: np.ndarray) -> np.ndarray:
    """Value of a 4-bit E2M1 code, bits [s e1 e0 m]: exponent bias 1, one
    mantissa bit, exponent field 0 is subnormal (0 or 0.5).  No inf/NaN."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(s == 1, -mag, mag)


def e8m0_value(byte: np.ndarray) -> np.ndarray:
    """Value of an E8M0 scale byte: 2^(s-127); 0xFF encodes NaN."""
    s = np.asarray(byte, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def mxfp4_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows -> float64 [R, K] ([A] 权重量化; format split per the
    OCP MX convention).  codes uint8 [R, K/2], scales uint8 [R, K/32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, half = codes.shape
    K = 2 * half
    assert scales.shape == (R, K // 32), (scales.shape, R, K)
    nib = np.empty((R, K), dtype=np.uint8)
    nib[:, 0::2] = codes & 0x0F          # element 2j: low nibble
    nib[:, 1::2] = codes >> 4            # element 2j+1: high nibble
    table = e2m1_value(np.arange(16))
    w = table[nib]
    scale = e8m0_value(scales)           # [R, K/32]
    return w * np.repeat(scale, 32, axis=1)


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, router_w: np.ndarray, router_b: np.ndarray) -> np.ndarray:
    """Router scores l[t, e] = sum_k x[t,k] W_r[e,k] + b_r[e] ([B] 2.4.1: a
    router scores every expert for each token).  x: float64 [T, d]."""
    return x @ router_w.T + router_b[None, :]


def topk_experts(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per row, descending; ties -> lower
    index ([A] 模型架构/MoE: top-4 routing).  int64 [T, k]."""
    T, E = logits.shape
    out = np.empty((T, k), dtype=np.int64)
    idx = np.arange(E)
    for t in range(T):
        order = np.lexsort((idx, -logits[t]))   # primary: -logit, secondary: index
        out[t] = order[:k]
    return out


def selected_softmax(sel_logits: np.ndarray) -> np.ndarray:
    """Softmax over the selected logits of each row ([A] 模型架构/MoE:
    softmax weighting of the chosen experts)."""
    m = sel_logits.max(axis=1, keepdims=True)
    e = np.exp(sel_logits - m)
    return e / e.sum(axis=1, keepdims=True)


def sigmoid(v: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-v))


def clamped_swiglu(g: np.ndarray, u: np.ndarray, clamp: float) -> np.ndarray:
    """h = Swish(clamp(g)) * (clamp(u) + 1): Swish(v) = v*sigmoid(v)
    ([A] Swish/SwiGLU 替换 GELU); gate-times-up GLU with a clamp and the
    residual-style +1 on the up branch ([A] 模型架构/MoE)."""
    gc = np.clip(g, -clamp, clamp)
    uc = np.clip(u, -clamp, clamp)
    return gc * sigmoid(gc) * (uc + 1.0)


ALT_SWISH_SLOPE = 1.702


def clamped_swiglu_alt(g: np.ndarray, u: np.ndarray, clamp: float) -> np.ndarray:
    """The alternative activation reading (the variant layout's): Swish with
    slope 1.702, v * sigmoid(1.702 v), on the gate clamped from above only,
    times the symmetrically clamped up branch plus one."""
    gc = np.minimum(g, clamp)
    uc = np.clip(u, -clamp, clamp)
    return gc * sigmoid(ALT_SWISH_SLOPE * gc) * (uc + 1.0)


def e2m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest FP6 E2M3 value (ties to the even code) of |v| <= 7.5: sign,
    two exponent bits (bias 1), three mantissa bits; the subnormals are
    m/8, the normals 2^(e-1) * (1 + m/8) for e = 1..3, so the spacing is 1/8
    below 2, 1/4 in [2, 4) and 1/2 in [4, 7.5].  Within a binade an even
    multiple of the spacing is an even mantissa, and round() breaks ties to
    even, so this is round-to-nearest-even on the codes."""
    a = np.abs(v)
    q = np.where(a < 2.0, 0.125, np.where(a < 4.0, 0.25, 0.5))
    return np.sign(v) * np.round(a / q) * q


def mx6_scale_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest integer k with 7.5 * 2^k >= amax (a block's shared E8M0
    exponent; 7.5 is the largest E2M3 value, so no element saturates).
    amax = 0 gives k = -127 (the block quantises to zeros)."""
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    k = np.ceil(np.log2(safe / 7.5))
    # settle the float rounding of log2 exactly: powers of two are exact
    k = np.where(7.5 * np.exp2(k - 1) >= safe, k - 1, k)
    k = np.where(7.5 * np.exp2(k) < safe, k + 1, k)
    return np.where(amax > 0, np.clip(k, -127, 127), -127.0)


def mxfp6_quantize(v: np.ndarray) -> np.ndarray:
    """Microscaling FP6 (E2M3 elements, one power-of-two scale per 32
    consecutive values of a row -- the same block format as the MXFP4
    weights of [A] 权重量化, with 6-bit elements): each block is divided by
    2^k (mx6_scale_exponent of its largest magnitude), rounded to E2M3,
    and multiplied back.  The activation-quantised fast mode feeds x and h
    through this before the expert GEMMs."""
    v = np.asarray(v, dtype=np.float64)
    shape = v.shape
    b = v.reshape(shape[:-1] + (shape[-1] // 32, 32))
    k = mx6_scale_exponent(np.abs(b).max(axis=-1))[..., None]
    s = np.exp2(k)
    return (e2m3_round(b / s) * s).reshape(shape)


def mx6x2_quantize(v: np.ndarray) -> np.ndarray:
    """Two-term microscaling FP6: the MXFP6 rounding of v (mxfp6_quantize)
    plus the MXFP6 rounding of what that leaves over, each 32-element block
    of each term with the scale of its own largest magnitude.  The reduced-
    precision option feeds x and h through this before the expert GEMMs
    (the exact path's activations carry a third such term)."""
    t0 = mxfp6_quantize(v)
    return t0 + mxfp6_quantize(np.asarray(v, dtype=np.float64) - t0)


def expert_ffn(xs: np.ndarray, w13: np.ndarray, b13: np.ndarray,
               w2: np.ndarray, b2: np.ndarray, clamp: float, act_quant=None, alt: bool = False) -> np.ndarray:
    """One expert on rows xs [n, d] with dequantised weights: the three
    linear maps of the GLU ([C]): a = xs W13^T + b13, gate = a[:, :I],
    up = a[:, I:], z = h W2^T + b2.  act_quant (fast mode only) is applied
    to the rows entering each expert GEMM (xs and h).  alt: the variant
    layout and activation -- gate and up rows interleaved (gate of column i
    in row 2i, up in row 2i + 1, b13 likewise) and clamped_swiglu_alt."""
    I = w13.shape[0] // 2
    if act_quant is not None:
        xs = act_quant(xs)
    a = xs @ w13.T + b13[None, :]
    if alt:
        h = clamped_swiglu_alt(a[:, 0::2], a[:, 1::2], clamp)
    else:
        h = clamped_swiglu(a[:, :I], a[:, I:], clamp)
    if act_quant is not None:
        h = act_quant(h)
    return h @ w2.T + b2[None, :]


def dequant_expert(experts: dict, e: int) -> tuple:
    """Expert e's weights in float64: (W13, b13, W2, b2)."""
    return (
        mxfp4_dequant(experts["w13_codes"][e], experts["w13_scales"][e]),
        np.asarray(experts["b13"][e], dtype=np.float64),
        mxfp4_dequant(experts["w2_codes"][e], experts["w2_scales"][e]),
        np.asarray(experts["b2"][e], dtype=np.float64),
    )


class DequantCache:
    """Dequantises expert e's weights on first use (float64) and keeps them
    (about 200 MB per expert at d = I = 2880)."""

    def __init__(self, experts: dict):
        self.ex = experts
        self._c: dict[int, tuple] = {}

    def __call__(self, e: int):
        if e not in self._c:
            self._c[e] = dequant_expert(self.ex, e)
        return self._c[e]


def route(x_bits: np.ndarray, router_w_bits: np.ndarray, router_b: np.ndarray, k: int):
    """Router, top-k and selected softmax.  Returns (logits, ids [T,k],
    weights [T,k])."""
    x = bf16_bits_to_f64(x_bits)
    wr = bf16_bits_to_f64(router_w_bits)
    logits = router_logits(x, wr, np.asarray(router_b, dtype=np.float64))
    ids = topk_experts(logits, k)
    w = selected_softmax(np.take_along_axis(logits, ids, axis=1))
    return logits, ids, w


def moe_layer(x_bits: np.ndarray, router_w_bits: np.ndarray, router_b: np.ndarray,
              experts: dict, k: int, clamp: float, cache: DequantCache | None = None,
              act: str = "exact", alt: bool = False):
    """Sparse MoE layer: y[t] = sum_j w[t,j] * FFN_{S_t[j]}(x[t]).

    Each expert runs only on the tokens routed to it ([B] 2.4.1).  Returns a
    dict with y (float64 [T, d]), logits, ids, w and per-expert counts.
    act = "mxfp6": the activation-quantised fast mode (x and h rounded to
    MXFP6 before the expert GEMMs, mxfp6_quantize); act = "mx6x2": the
    two-term option (mx6x2_quantize); the router always sees x.
    alt: the variant weight layout and activation of expert_ffn.
    """
    if act not in ("exact", "mxfp6", "mx6x2"):
        raise ValueError(act)
    aq = {"exact": None, "mxfp6": mxfp6_quantize, "mx6x2": mx6x2_quantize}[act]
    x = bf16_bits_to_f64(x_bits)
    logits, ids, w = route(x_bits, router_w_bits, router_b, k)
    T = x.shape[0]
    E = router_w_bits.shape[0]
    d = x.shape[1]
    # without a cache each expert is dequantised for its own tokens and
    # dropped afterwards, so memory stays at one expert
    get = cache if cache is not None else (lambda e: dequant_expert(experts, e))
    y = np.zeros((T, d), dtype=np.float64)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    for e in range(E):
        tok, slot = np.nonzero(ids == e)
        if tok.size == 0:
            continue
        w13, b13, w2, b2 = get(e)
        z = (expert_ffn(x[tok], w13, b13, w2, b2, clamp) if aq is None and not alt
             else expert_ffn(x[tok], w13, b13, w2, b2, clamp, aq, alt))
        y[tok] += w[tok, slot][:, None] * z
    return dict(y=y, logits=logits, ids=ids, w=w, counts=counts)


def moe_layer_dense_masked(x_bits: np.ndarray, router_w_bits: np.ndarray, router_b: np.ndarray,
                           experts: dict, k: int, clamp: float) -> np.ndarray:
    """Brute-force form of the same layer for tiny inputs: run every expert
    on every token, then mix with a mask that is w[t,e] on the selected
    experts and 0 elsewhere.  Written independently of moe_layer (no shared
    routing helper): the mask comes from a full sort and a full softmax
    renormalised over the selected set."""
    x = bf16_bits_to_f64(x_bits)
    wr = bf16_bits_to_f64(router_w_bits)
    b = np.asarray(router_b, dtype=np.float64)
    T, d = x.shape
    E = wr.shape[0]
    y = np.zeros((T, d))
    for t in range(T):
        l = np.array([float(np.dot(x[t], wr[e])) + b[e] for e in range(E)])
        ranked = sorted(range(E), key=lambda e: (-l[e], e))
        chosen = set(ranked[:k])
        p = np.exp(l - l.max())
        p = p / p.sum()
        zsum = sum(p[e] for e in chosen)
        for e in range(E):
            mask = p[e] / zsum if e in chosen else 0.0
            w13 = mxfp4_dequant(experts["w13_codes"][e], experts["w13_scales"][e])
            w2 = mxfp4_dequant(experts["w2_codes"][e], experts["w2_scales"][e])
            I = w13.shape[0] // 2
            g = np.array([np.dot(w13[i], x[t]) for i in range(I)]) + experts["b13"][e][:I]
            u = np.array([np.dot(w13[I + i], x[t]) for i in range(I)]) + experts["b13"][e][I:]
            gc = np.minimum(np.maximum(g, -clamp), clamp)
            uc = np.minimum(np.maximum(u, -clamp), clamp)
            h = gc / (1.0 + np.exp(-gc)) * (1.0 + uc)
            z = np.array([np.dot(w2[r], h) for r in range(d)]) + experts["b2"][e]
            y[t] += mask * z
    return y


def rmsnorm(v: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) over the last axis, unit gain, no bias
    ([A] RMSNorm 替换 LayerNorm)."""
    return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)


def stack_forward(x0_bits: np.ndarray, layers: list, k: int, clamp: float, eps: float = 1e-5):
    """Pre-norm residual stack of MoE layers: n = bf16(RMSNorm(x)),
    x <- bf16(x + MoE(n)).  ``layers`` is a list of dicts with router_w,
    router_b and the expert arrays.  Returns the final residual stream
    (float64 holding bf16 values) and the per-layer ids."""
    x = bf16_bits_to_f64(x0_bits)
    all_ids = []
    for L in layers:
        n = round_to_bf16(rmsnorm(x, eps))
        n_bits = _f64_bf16_to_bits(n)
        r = moe_layer(n_bits, L["router_w"], L["router_b"], L, k, clamp)
        all_ids.append(r["ids"])
        x = round_to_bf16(x + r["y"])
    return x, all_ids


def _f64_bf16_to_bits(v: np.ndarray) -> np.ndarray:
    """Bit pattern of float64 values that are already bf16-representable."""
    f = np.asarray(v, dtype=np.float32)          # exact for bf16 values
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def topk_gap(logits: np.ndarray, k: int) -> np.ndarray:
    """Gap between the k-th and (k+1)-th largest logit of each row (inf when
    k equals the number of experts).  The top-k set of a row is decided by
    that gap: a perturbation of every logit by less than half of it leaves
    the set unchanged."""
    s = -np.sort(-logits, axis=1)
    if s.shape[1] <= k:
        return np.full(s.shape[0], np.inf)
    return s[:, k - 1] - s[:, k]
