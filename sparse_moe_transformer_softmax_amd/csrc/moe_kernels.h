// Kernel parameter blocks and host-side launchers of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

struct RouteParams {
  const uint16_t* x;         // bf16 [T, d]
  const uint16_t* router_w;  // bf16 [E, d]
  const float* router_b;     // fp32 [E]
  int T, d, E, k, mt;        // mt: rows per GEMM tile
  int* topk_id;              // [T, k]
  float* topk_w;             // [T, k]
  int* rel_pos;              // [T, k] row of the pair inside its expert's list
  int* expert_rows;          // [E, T] pair ids (t*k + j) per expert
  int* cursor;               // [256 * CURSOR_STRIDE], expert e at e * CURSOR_STRIDE; zero between calls
  int* done;                 // zero between calls
  int* counts;               // [E]
  int* offsets;              // [E + 1]
  int* n_tiles;              // [1]
  int2* tiles;               // [max_tiles] (expert, first row)
  // K split over workgroups (set by launch_route)
  int n_tb, ks;              // token blocks, workgroups per token block
  float* part;               // [n_tb * ks * 16 * mbr][E] partial logits (route_partial_bytes)
  int* tb_done;              // [ROUTE_MAX_TB * CURSOR_STRIDE] zero between calls
  uint8_t* xq;               // MX6x3 rows of x [T, d/32, 80], or null (no split)
  int* fold_cnt;             // [n_fold] arrival counters of the combine folded into the down
  int n_fold;                //   GEMM, zeroed by the trailing workgroups (null: no fold)
};

struct GemmParams {
  const int* n_tiles;
  const int2* tiles;
  const int* counts;
  const int* offsets;
  const int* expert_rows;    // gate/up only: [E, T]
  int T, k;
  const uint8_t* a;          // MX6x3 rows: token rows (gate/up) or permuted pair rows (down)
  const uint8_t* b_codes;    // [E, N, K/2]
  const uint8_t* b_scales;   // [E, N, K/32]
  const float* bias;         // [E, N]
  int N, K, I, E;
  float clamp;
  uint8_t* hq;               // gate/up output: MX6x3 rows [P, I/32, 80]
  float* y;                  // down output: fp32 [P, N]
  int terms;                 // FP6 terms of A taking part: 3 (exact path) or 1 (fast mode)
  int mb;                    // decode only: 16-row A blocks per tile (1, or 2 for 32-row tiles)
  int packed;                // wide prefill kernel only: 1 = weights in the packed layout (moe_pack_weights)
  int alt;                   // gate/up only: 1 = the variant layout and activation (interleaved rows,
                             // Swish slope 1.702, gate clamped from above only)
  // down, decode only: the combine folded into the epilogue (fold_cnt null: no fold)
  int* fold_cnt;             // [T, ceil(N/64)] arrivals per (token, 64-column span), zero at launch
  int* pair_row;             // [T, k] row of y holding each (token, slot) pair: written by the
                             //   gate/up decode launch, read by the fold (null: no fold)
  const float* topk_w;       // [T, k]
  uint16_t* out;             // bf16 [T, N]
  float* out_f32;            // fp32 [T, N] or null
};

struct CombineParams {
  const float* y;            // [P, d] permuted expert outputs (bias included)
  const int* topk_id;
  const float* topk_w;
  const int* rel_pos;
  const int* offsets;
  int T, d, k;
  uint16_t* out;             // bf16 [T, d] or null
  float* out_f32;            // fp32 [T, d] or null
  // residual stack variant (all null otherwise)
  const uint16_t* resid_in;  // bf16 [T, d]
  uint16_t* resid_out;       // bf16 [T, d]  = bf16(resid_in + sum)
  uint16_t* norm_out;        // bf16 [T, d]  = bf16(rmsnorm(resid_out))
  float eps;
};

int launch_route(const RouteParams& p, hipStream_t s);
// GEMM configurations: decode (16-row tiles), prefill (64-row tiles),
// wide prefill (128-row tiles)
enum GemmMode { GEMM_DECODE = 0, GEMM_PREFILL = 1, GEMM_WIDE = 2, GEMM_WIDE64 = 3 };
// Optional events that a launch records itself when its kernel starts and
// ends (timing of one kernel without the dispatch before it).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
int launch_gemm_gateup(const GemmParams& p, int max_tiles, int mode, hipStream_t s, const LaunchEvents& ev = {});
int launch_gemm_down(const GemmParams& p, int max_tiles, int mode, hipStream_t s, const LaunchEvents& ev = {});
int launch_combine(const CombineParams& p, hipStream_t s);
int launch_rmsnorm(const uint16_t* x, uint16_t* out, int T, int d, float eps, hipStream_t s);
int launch_residual_rmsnorm(const uint16_t* x, const void* y, bool y_f32, uint16_t* x_out, uint16_t* n_out, int T,
                            int d, float eps, hipStream_t s);
int launch_zero_ints(int* p, int n, hipStream_t s);

// ints between consecutive expert cursors (one 128-byte cache line)
constexpr int CURSOR_STRIDE = 32;
// most token blocks whose K range the router splits over workgroups (one
// arrival counter each), and the workgroups it aims for
constexpr int ROUTE_MAX_TB = 256;
constexpr int ROUTE_TARGET_WG = 256;
// bytes of partial logits the router's K split exchanges for T tokens over E
// experts (0: no split)
size_t route_partial_bytes(int T, int E);

// K sub-slices of a router workgroup's 16 waves: 16 / (its expert groups),
// fewer where the LDS partials (sub-slices x 16 * mbr tokens x (16 * ncb + 1)
// floats) would not fit 16 * 1032 floats
__host__ __device__ inline int route_wave_kslices(int ncb, int ncbw, int mbr) {
  const int eg = (ncb + ncbw - 1) / ncbw;
  int ks = 16 / eg;
  while (ks > 1 && ks * 16 * mbr * (16 * ncb + 1) > 16 * 1032) --ks;
  return ks;
}

// rows per GEMM tile of the two configurations
constexpr int MT_SMALL = 16;
constexpr int MT_SMALL2 = 32;  // decode tiles of two row blocks
constexpr int MT_LARGE = 64;
constexpr int MT_WIDE = 128;

// Attention beside the layer: q bf16 [B, Tq, Hq, D], k and v bf16 [B, S, Hkv, D],
// out bf16 [B, Tq, Hq, D], D = 64; query i at position q_pos0 + i.
struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* sinks;        // [Hq] sink logits
  uint16_t* out;
  int B, Tq, S, q_pos0, Hq, Hkv;
  int window;                // 0: dense causal; otherwise the band of the last `window` positions
  float qk_scale;            // log2(e) / sqrt(D)
};
int launch_attention(const AttnParams& p, hipStream_t s);
int attn_positions_per_wave(int G);
int launch_rope(const uint16_t* x, uint16_t* out, int n, int H, int D, int pos0, float theta, hipStream_t s);
// Packs one stack of MXFP4 matrices ([E, N, K/2] codes, [E, N, K/32] scales)
// into the layout of the wide prefill kernel (see moe_pack_weights).
int launch_pack_weights(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* codes_out,
                        uint8_t* scales_out, hipStream_t s);

}  // namespace moe
