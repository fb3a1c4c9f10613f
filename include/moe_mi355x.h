/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) gpt-oss mixture-of-experts
 * MLP layer.
 *
 * The layer (gpt-oss pages: "OpenAI 最新开源模型 gpt-oss 架构与训练解析",
 * 模型架构 section, MoE item; "【LLM】GPT-OSS架构变化详解", 2.4.1):
 *   logits[t, e] = x[t] . W_r[e] + b_r[e]                       (router)
 *   S_t          = the k experts with the largest logits         (top-k)
 *   w[t, j]      = softmax over the k selected logits            (gate weights)
 *   a            = W13_e x[t] + b13_e ; g = a[0:I], u = a[I:2I]
 *   h            = clamp(g) * sigmoid(clamp(g)) * (clamp(u) + 1) (clamped SwiGLU)
 *   z            = W2_e h + b2_e                                 (down projection)
 *   out[t]       = sum_j w[t, j] * z_{S_t[j]}                    (combine)
 * clamp(v) limits v to [-clamp, clamp].  The expert weights are MXFP4
 * (same page, 权重量化 item: 4.25 bits per weight): E2M1 codes, two per byte
 * with the low nibble holding the even element, and one E8M0 scale byte
 * (value 2^(s-127), 0xFF = NaN) per 32 consecutive elements of a row.
 *
 * Conventions shared by every entry point:
 *  - All array arguments are DEVICE pointers on the current HIP device,
 *    row-major and contiguous.  bf16 arrays are passed as raw 16-bit
 *    patterns.  x, router_w, out and the code and scale arrays must be
 *    16-byte aligned; fp32 arrays 4-byte aligned.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *    enqueued asynchronously; the library never synchronises the stream,
 *    so device faults surface at the caller's next synchronisation.
 *  - The caller owns every buffer it passes; the library keeps no pointer
 *    after a call returns.
 *  - Return value: MOE_OK (0) or a negative moe_status.  No C++ exception
 *    crosses the boundary and the library prints nothing.
 *  - Shapes: T >= 0 tokens (T == 0 is a successful no-op); d (model width)
 *    and I (expert width) positive multiples of 32; 1 <= E <= 256 experts;
 *    1 <= k <= min(E, 8); T * max(k, E) < 2^31; clamp > 0 (+inf disables
 *    the clamp).  Larger problems than the kernels address with 32-bit
 *    offsets return MOE_ERR_UNSUPPORTED: T * k * max(d, I) * 5/2 must stay
 *    below 2^31 bytes (the activation operand) and E * I * d below 2^32
 *    (the gate/up weight codes).
 *  - Entry points without a workspace argument use a library-owned device
 *    workspace per GPU that grows on demand (a growth allocates and
 *    synchronises the device).  Calls that share it must be ordered on one
 *    stream; concurrent callers pass their own workspace to
 *    moe_layer_forward_ws.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MI355X_VERSION 10000 /* 1.0.0 */

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
  MOE_ERR_BAD_SHAPE = -2,   /* a size is out of range or inconsistent */
  MOE_ERR_UNSUPPORTED = -3, /* no gfx950 device is current, or the problem is too large */
  MOE_ERR_MISALIGNED = -4,  /* a pointer breaks the alignment rules above */
  MOE_ERR_NOMEM = -5,       /* workspace allocation failed */
  MOE_ERR_HIP = -6,         /* a HIP launch or runtime call failed */
  MOE_ERR_ALIAS = -7,       /* the output overlaps an input */
  MOE_ERR_WORKSPACE = -8    /* caller workspace too small */
} moe_status;

/* Full MoE layer.
 *   x          bf16 [T, d]            token activations
 *   router_w   bf16 [E, d]            router weight
 *   router_b   fp32 [E]               router bias
 *   w13_codes  uint8 [E, 2I, d/2]     fused gate/up weight, E2M1 nibbles;
 *                                     rows [0, I) gate, rows [I, 2I) up
 *   w13_scales uint8 [E, 2I, d/32]    E8M0 scales of w13
 *   b13        fp32 [E, 2I]           gate/up bias
 *   w2_codes   uint8 [E, d, I/2]      down weight, E2M1 nibbles
 *   w2_scales  uint8 [E, d, I/32]     E8M0 scales of w2
 *   b2         fp32 [E, d]            down bias (inside the expert, so it
 *                                     is weighted by the gate weight)
 *   out        bf16 [T, d]            written; must not overlap any input
 * Top-k ties go to the lower expert index. */
int moe_layer_forward(const void* x, const void* router_w, const float* router_b,
                      const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                      const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2,
                      int T, int d, int I, int E, int k, float clamp, void* out, void* stream);

/* Same kernels as moe_layer_forward, with the intermediate results exposed.
 *   out      bf16 [T, d] or NULL
 *   out_f32  fp32 [T, d] or NULL: the combine result before bf16 rounding
 *            (out == round-to-nearest-even(out_f32) element by element)
 *   topk_id  int32 [T, k]  selected experts, descending logit
 *   topk_w   fp32 [T, k]   their softmax weights
 *   counts   int32 [E]     number of (token, slot) pairs per expert
 * topk_id, topk_w and counts are required. */
int moe_layer_forward_dbg(const void* x, const void* router_w, const float* router_b,
                          const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                          const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2,
                          int T, int d, int I, int E, int k, float clamp, void* out, float* out_f32,
                          int32_t* topk_id, float* topk_w, int32_t* counts, void* stream);

/* Activation-quantised fast mode of moe_layer_forward (same arguments,
 * layouts, ownership and errors).  The rows entering each expert GEMM (x
 * for gate/up, h for down) are rounded to MXFP6 -- E2M3 elements with one
 * power-of-two scale per 32 consecutive values, the smallest scale 2^k with
 * 7.5 * 2^k >= the block's largest magnitude, round-to-nearest-even -- the
 * block format of the pages' MXFP4 weights ("OpenAI 最新开源模型 gpt-oss
 * 架构与训练解析", 权重量化 item) with 6-bit elements.  One block-scaled
 * MFMA per 128-wide K step instead of three.  The router sees x unrounded,
 * so expert ids and weights equal moe_layer_forward's.  The result is that
 * of the layer on the rounded activations, not of the exact layer: it
 * differs from moe_layer_forward by a few per cent of rms. */
int moe_layer_forward_mx6(const void* x, const void* router_w, const float* router_b,
                          const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                          const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2,
                          int T, int d, int I, int E, int k, float clamp, void* out, void* stream);

/* moe_layer_forward_dbg for the fast mode (outputs as there). */
int moe_layer_forward_mx6_dbg(const void* x, const void* router_w, const float* router_b,
                              const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                              const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2,
                              int T, int d, int I, int E, int k, float clamp, void* out, float* out_f32,
                              int32_t* topk_id, float* topk_w, int32_t* counts, void* stream);

/* Flags of moe_layer_forward_ex. */
enum moe_layer_flags {
  /* the activation-quantised fast mode of moe_layer_forward_mx6 */
  MOE_LAYER_MXFP6 = 1,
  /* the variant activation reading: h = g' * sigmoid(1.702 g') * (u' + 1)
   * with g' = min(g, clamp) (the gate clamped from above only) and
   * u' = clamp(u, -clamp, clamp); and the variant weight layout of
   * w13_codes / w13_scales / b13: gate and up rows interleaved, row 2i the
   * gate of output column i and row 2i+1 its up (b13 likewise).  The pages
   * give Swish with unit slope and a clamp without its placement
   * ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", MoE item and Swish/SwiGLU
   * 替换 GELU); this flag selects the other reading of both. */
  MOE_LAYER_ALT_ACT = 2,
  /* the expert weights (w13_codes, w13_scales, w2_codes, w2_scales) are in
   * the packed layout written by moe_pack_weights; biases unchanged.  d and
   * I must be multiples of 64 (otherwise MOE_ERR_UNSUPPORTED).  Results are
   * bitwise those of the row-major weights. */
  MOE_LAYER_PACKED = 4,
  /* the two-term option: the rows entering each expert GEMM are rounded to
   * two MXFP6 terms -- the MXFP6 rounding of the row (as in the fast mode)
   * plus the MXFP6 rounding of what it leaves over, each 32-block of each
   * term with its own power-of-two scale -- instead of the exact path's
   * three: two block-scaled MFMAs per 128-wide K step instead of three.
   * Each value is then within 1/225 of its block's largest magnitude; the
   * layer differs from moe_layer_forward by about 1e-3 of its rms (at most
   * 5e-3 to 8e-3 in the cases measured, against 0.3-0.4 for the one-term
   * fast mode).  The router sees x unrounded.  Not together with
   * MOE_LAYER_MXFP6 (MOE_ERR_BAD_SHAPE). */
  MOE_LAYER_MX6X2 = 8
};

/* moe_layer_forward with flags (any OR of moe_layer_flags; unknown bits give
 * MOE_ERR_BAD_SHAPE).  topk_id, topk_w and counts are all null or all set
 * (as in moe_layer_forward_dbg); out_f32 may be set only with them. */
int moe_layer_forward_ex(const void* x, const void* router_w, const float* router_b,
                         const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                         const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2,
                         int T, int d, int I, int E, int k, float clamp, int flags, void* out,
                         float* out_f32, int32_t* topk_id, float* topk_w, int32_t* counts, void* stream);

/* Router, top-k and selected softmax only ("【LLM】GPT-OSS架构变化详解",
 * 2.4.1; "OpenAI 最新开源模型 gpt-oss 架构与训练解析", MoE item).  Outputs as
 * in moe_layer_forward_dbg. */
int moe_route(const void* x, const void* router_w, const float* router_b, int T, int d, int E,
              int k, int32_t* topk_id, float* topk_w, int32_t* counts, void* stream);

/* Bytes of device workspace moe_layer_forward_ws needs for these sizes
 * (0 if the sizes are invalid). */
size_t moe_workspace_bytes(int T, int d, int I, int E, int k);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the layer
 * of moe_layer_forward (same arguments, layouts, results and errors) with
 * its scratch in a static device array of MOE_NOALLOC_SCRATCH_BYTES that
 * every GPU the library runs on holds until the process ends.  The call
 * allocates nothing (no hipMalloc or hipFree, no library allocation); it
 * launches one small kernel that clears the array's counters, then the
 * layer.  Sizes whose workspace (moe_workspace_bytes) exceeds the array
 * return MOE_ERR_WORKSPACE -- about 800 tokens at d = I = 2880, k = 4.
 * All calls on one GPU share its array: calls that overlap in time on one
 * GPU (different streams, or different host threads) race and must not be
 * issued; calls on one stream are ordered and safe. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_layer_forward_noalloc(const void* x, const void* router_w, const float* router_b,
                              const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                              const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2, int T, int d, int I,
                              int E, int k, float clamp, void* out, void* stream);

/* Prepares a caller-owned workspace (256-byte aligned, at least
 * moe_workspace_bytes) for first use by clearing its counter block with a
 * kernel on `stream`.  Every completed call leaves the block cleared again. */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward with a caller-owned workspace: allocates nothing.
 * Concurrent calls need distinct workspaces. */
int moe_layer_forward_ws(const void* x, const void* router_w, const float* router_b,
                         const uint8_t* w13_codes, const uint8_t* w13_scales, const float* b13,
                         const uint8_t* w2_codes, const uint8_t* w2_scales, const float* b2,
                         int T, int d, int I, int E, int k, float clamp, void* out, void* ws,
                         size_t ws_bytes, void* stream);

/* out = bf16(x / sqrt(mean(x^2) + eps)) per row, unit gain, no bias
 * ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", RMSNorm 替换 LayerNorm).
 * x, out bf16 [T, d]; d a multiple of 32; eps >= 0.  out may equal x. */
int moe_rmsnorm(const void* x, void* out, int T, int d, float eps, void* stream);

/* The residual add and RMSNorm between two layers of the stack, fused
 * ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", RMSNorm 替换 LayerNorm: a
 * pre-norm block adds its output to the residual stream, and the next
 * block normalises that stream by its root mean square, unit gain):
 *   x_out = bf16(x + y)                                  (the add in fp32)
 *   n_out = bf16(x_out / sqrt(mean(x_out^2) + eps))      (per row)
 *   x      bf16 [T, d]   residual stream
 *   y_bf16 bf16 [T, d]   layer output, or NULL
 *   y_f32  fp32 [T, d]   layer output, or NULL (exactly one of the two is set;
 *                        the fp32 form is what moe_layer_forward_dbg returns
 *                        as out_f32, and what the stack adds internally)
 *   x_out  bf16 [T, d]   written; may be x itself, otherwise must not overlap
 *                        x, y or n_out
 *   n_out  bf16 [T, d]   written, or NULL (residual add only); must not
 *                        overlap x, y or x_out
 * d a multiple of 32 and eps >= 0.  Sums of squares are taken over the
 * rounded x_out values, in fp32. */
int moe_rmsnorm_residual(const void* x, const void* y_bf16, const float* y_f32, void* x_out, void* n_out, int T,
                         int d, float eps, void* stream);

/* Repacks one stack of MXFP4 matrices, as stored ("OpenAI 最新开源模型 gpt-oss
 * 架构与训练解析", 权重量化 item): codes u8 [E, N, K/2] (two E2M1 codes per
 * byte, row-major) and scales u8 [E, N, K/32] (E8M0), into the layout the
 * prefill GEMM streams whole 128-byte lines of (MOE_LAYER_PACKED):
 *   codes_out  u8 [E, N/2, K]: for each pair of weight rows (2p, 2p+1) and
 *              each chunk c of four 32-element blocks (64 bytes of a row),
 *              row 2p's chunk bytes then row 2p+1's (a last chunk of two
 *              blocks keeps 32 + 32 bytes); E * N * K/2 bytes in all
 *   scales_out u8 [E, ceil(K/128), N, 4]: for each chunk c, the four scale
 *              bytes of blocks 4c .. 4c+3 of every row, rows consecutive
 *              (blocks past K/32 hold 127); moe_packed_scale_bytes bytes
 * Call it once per weight matrix (W13 with N = 2I, K = d; W2 with N = d,
 * K = I).  N even and K a multiple of 64; codes and codes_out 16-byte
 * aligned, scales_out 4-byte aligned; outputs must not overlap the inputs
 * or each other.  Byte values are copied unchanged. */
int moe_pack_weights(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* codes_out,
                     uint8_t* scales_out, void* stream);

/* Bytes of moe_pack_weights' scales_out for these sizes (0 if invalid). */
size_t moe_packed_scale_bytes(int E, int N, int K);

/* Pre-norm residual stack of n_layers MoE layers on one GPU:
 *   n = bf16(RMSNorm(x)); x = bf16(x + MoE_l(n))   for l = 0 .. n_layers-1
 * Each per-layer argument is a HOST array of n_layers device pointers with
 * the layouts of moe_layer_forward.  x0 bf16 [T, d] is read; out bf16 [T, d]
 * receives the final residual stream and must not overlap x0. */
int moe_stack_forward(const void* x0, int n_layers, const void* const* router_w,
                      const float* const* router_b, const uint8_t* const* w13_codes,
                      const uint8_t* const* w13_scales, const float* const* b13,
                      const uint8_t* const* w2_codes, const uint8_t* const* w2_scales,
                      const float* const* b2, int T, int d, int I, int E, int k, float clamp,
                      float eps, void* out, void* stream);

/* moe_stack_forward with flags: MOE_LAYER_ALT_ACT and MOE_LAYER_PACKED (the
 * per-layer expert weights in the packed layout); other bits give
 * MOE_ERR_BAD_SHAPE. */
int moe_stack_forward_ex(const void* x0, int n_layers, const void* const* router_w, const float* const* router_b,
                         const uint8_t* const* w13_codes, const uint8_t* const* w13_scales, const float* const* b13,
                         const uint8_t* const* w2_codes, const uint8_t* const* w2_scales, const float* const* b2,
                         int T, int d, int I, int E, int k, float clamp, float eps, int flags, void* out,
                         void* stream);

/* ------------------------------------------------------------------------
 * The attention steps beside the layer ("OpenAI 最新开源模型 gpt-oss 架构与训练
 * 解析", 模型架构: Attention item -- grouped-query attention with 64 query
 * heads over 8 key/value heads, layers alternating between a band of the
 * last 128 positions and dense attention, rotary position encoding, and a
 * learned per-head bias logit in the softmax denominator; same page,
 * "RoPE 替换了绝对位置编码" and "Attention Bias and Attention Sinks").
 * The projections that produce q, k and v (and the output projection) are
 * plain dense GEMMs and are not part of this library.
 * ------------------------------------------------------------------------ */

/* Rotary position encoding of n rows of H heads of width D:
 *   out[t, h, 2i]   = x[t, h, 2i] cos(a) - x[t, h, 2i+1] sin(a)
 *   out[t, h, 2i+1] = x[t, h, 2i] sin(a) + x[t, h, 2i+1] cos(a)
 * with a = (pos0 + t) * theta^(-2i/D) (theta = 10000 in the workloads).  x,
 * out bf16 [n, H, D], 16-byte aligned; out may equal x (in place), otherwise
 * must not overlap it.  D even, 2 <= D <= 256; n, H >= 0 (0 is a no-op);
 * pos0 >= 0, pos0 + n < 2^31; theta > 1.  The angle is formed in double
 * precision; the rotation is fp32, rounded once to bf16. */
int moe_attn_rope(const void* x, void* out, int n, int H, int D, int pos0, float theta, void* stream);

/* Attention of B sequences, each with Tq queries at positions
 * q_pos0 .. q_pos0 + Tq - 1 over S keys at positions 0 .. S - 1:
 *   s_j    = q . k_j / sqrt(D)               for keys j the query sees:
 *            j <= p (causal), and p - j < window when window > 0
 *   out    = sum_j e^(s_j) v_j / (sum_j e^(s_j) + e^(sinks[h]))
 * Query head h reads key/value head h / (Hq / Hkv).
 *   q      bf16 [B, Tq, Hq, D]   (rotary encoding already applied)
 *   k, v   bf16 [B, S, Hkv, D]   (k with rotary encoding applied)
 *   sinks  fp32 [Hq]             sink logit of each query head (on the scale
 *                                of s_j; -inf removes it)
 *   out    bf16 [B, Tq, Hq, D]   written; must not overlap q, k, v or sinks
 * D == 64; Hq a multiple of Hkv with Hq / Hkv in {1, 2, 4, 8, 16}; B and Hkv
 * at most 65535 (larger values return MOE_ERR_UNSUPPORTED); B, Tq >= 0
 * (0 is a no-op); S >= 1; 0 <= q_pos0 and q_pos0 + Tq <= S; window >= 0
 * (0 = dense).  q, k, v and out 16-byte aligned, sinks 4-byte aligned.
 * Unsupported widths or group sizes return MOE_ERR_UNSUPPORTED, other bad
 * sizes MOE_ERR_BAD_SHAPE.  Scores and the softmax are fp32, the products
 * run on bf16 MFMAs with fp32 accumulation, and the output is rounded once
 * to bf16.  The result does not depend on timing. */
int moe_attn_forward(const void* q, const void* k, const void* v, const float* sinks, void* out, int B, int Tq,
                     int S, int q_pos0, int Hq, int Hkv, int D, int window, void* stream);

/* Per-kernel timing for profiling.  Bit i of mask selects kernel kind i of
 * {0 route (including the MX6x3 split of x, done by the same launch),
 * 1 gate/up GEMM, 2 down GEMM, 3 combine, 4 reserved (never launched)};
 * single-layer calls at decode sizes (T * k <= 16 * E) fold the combine
 * into the down GEMM, and then launch no kind 3 kernel;
 * while a kind is selected, every layer call records a HIP event pair
 * around each launch of that kernel on the call's stream (mask 0 turns
 * timing off; 0x1f times every kernel).  moe_timing_read waits for the
 * recorded events, fills ms[5] with the summed milliseconds and
 * launches[5] with the launch counts of the kinds above since the last
 * reset, and resets the sums when reset != 0.  Not thread-safe. */
int moe_timing_enable(int mask);
int moe_timing_read(double* ms, int* launches, int reset);

/* Frees the library-owned workspaces (waits for the device first). */
void moe_release(void);

/* Static description of a status code. */
const char* moe_status_string(int status);

/* MOE_MI355X_VERSION of the loaded library. */
int moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
