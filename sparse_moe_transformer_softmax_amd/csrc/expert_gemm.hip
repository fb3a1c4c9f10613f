// Expert-grouped GEMMs on the CDNA4 block-scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, A = FP6 E2M3, B = FP4 E2M1).
//
// Gate/up projection with the fused clamped-SwiGLU epilogue, and the down
// projection, of the gpt-oss MoE experts ("OpenAI 最新开源模型 gpt-oss 架构与
// 训练解析", 模型架构: MoE item, gated SwiGLU with clamp and the +1 on the up
// branch; Xin Zhiyuan's translation of Raschka, GLU section: three linear
// layers per expert; 权重量化 item: MXFP4 expert weights).
//
// The MXFP4 weights are the B operand and are fed to the MFMA as stored:
// each lane loads the 16 bytes (32 codes) of one 32-element block of one
// weight row and passes that block's E8M0 byte as its scale.  The
// activations are the A operand, stored as MX6x3 rows (three FP6 terms, one
// E8M0 scale each, per 32-element block); every 16x16x128 step issues one
// MFMA per term into the same fp32 accumulator.
//
// Operand layout of the 16x16x128 scaled MFMA (checked bit for bit by the
// one-hot layout probe tests, in every tile configuration): lane l carries row (A) or column (B) l % 16 and the 32
// consecutive K values of block l / 16 of the 128-wide step; the result
// C[4*(l/16) + q][l % 16] sits in accumulator element q of lane l.
//
// Work decomposition: the router's tile list (expert, first row) times
// spans of output columns.  Gate/up workgroups own matching gate and up
// columns, so the epilogue has both halves of h in the same lane.
#include <algorithm>
#include <type_traits>

#include <hip/hip_ext.h>

#include "moe_common.h"
#include "moe_kernels.h"

// The folded combine's cross-workgroup ordering relies on gfx950's cache
// behaviour for agent-scope atomic stores and loads (see the down
// projection's epilogue).
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "expert_gemm.hip is written for gfx950 only"
#endif

namespace moe {

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1: array indices
// stay compile-time constants, so register arrays never fall back to
// private memory.
template <int I, int N>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    if constexpr (I < N) {
      f(std::integral_constant<int, I>{});
      StaticFor<I + 1, N>::run(f);
    }
  }
};

// clamp(g) * sigmoid(clamp(g)) * (clamp(u) + 1) with the hardware exp2 and
// reciprocal (a few ulp; the result is then rounded to 2^-13 of its block
// maximum by the MX6x3 split).  The clamp to [-c, c] (c > 0, +inf allowed)
// is the median of (v, -c, c), equal to min(max(v, -c), c) for every
// non-NaN v, signed zeros included; a NaN in g or u (one unordered
// compare) makes the result NaN.  Without a clamp, large |g| gives the
// limits 0 and g (exp2 overflows to inf, its reciprocal to 0).
// The variant activation reading (alt) differs only in two constants: Swish
// with slope 1.702 on the gate clamped from above only (the median of (g,
// -inf, c)), times the symmetrically clamped up plus one.  glo and gk are
// the gate's lower bound and the exponent's factor of either reading
// (swiglu_consts), so the function has no branch.
struct SwigluConsts {
  float glo, gk;
};
__device__ __forceinline__ SwigluConsts swiglu_consts(float c, int alt) {
  return alt ? SwigluConsts{-__builtin_inff(), 1.702f * 1.44269504088896341f}
             : SwigluConsts{-c, 1.44269504088896341f};
}
__device__ __forceinline__ float clamped_swiglu(float g, float u, float c, SwigluConsts k) {
  const float gc = __builtin_amdgcn_fmed3f(g, k.glo, c);
  const float uc = __builtin_amdgcn_fmed3f(u, -c, c);
  const float e = __builtin_amdgcn_exp2f(-gc * k.gk);
  const float h = gc * __builtin_amdgcn_rcpf(1.0f + e) * (uc + 1.0f);
  return __builtin_isunordered(g, u) ? g + u : h;
}

__device__ __forceinline__ float swiglu_act(float g, float u, float c, int alt) {
  return clamped_swiglu(g, u, c, swiglu_consts(c, alt));
}

// Row of the fused gate/up weight (and index of its bias) that holds output
// column c of the gate (up = 0) or up (up = 1) projection: gate rows then up
// rows, or (the variant layout) interleaved, gate of column c in row 2c.
__device__ __forceinline__ int gu_row(int c, int up, int I, int alt) { return alt ? 2 * c + up : up * I + c; }

template <int MB, int NCB>
struct Stage {
  uint4 a[MB][5];  // MX6x3 block of each 16-row block (3 x 24 B codes, 3 scale bytes)
  uint4 bc[NCB];   // 32 E2M1 codes of each weight column block
  int bs[NCB];     // E8M0 scale of each weight column block
};

// One 128-wide K step for every (row block, column block): three MFMAs,
// one per FP6 term of A.  keep = 0 on lanes whose K block does not take
// part (past the end of K or outside the wave's share): they contribute
// zero codes with a unit scale.
template <int MB, int NCB>
__device__ __forceinline__ uint32_t keep_mask(bool in) { return in ? 0xffffffffu : 0u; }

// TERMS = 1 (the activation-quantised fast mode): only the first FP6 term
// of A takes part; TERMS = 2 (the two-term option): the first two.
template <int MB, int NCB, int TERMS = 3>
__device__ __forceinline__ void mma_stage(v4f (&acc)[MB][NCB], const Stage<MB, NCB>& st, uint32_t keep) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const uint32_t* aw = (const uint32_t*)&st.a[mb][0];
    const v8i a0 = {(int)aw[0], (int)aw[1], (int)aw[2], (int)aw[3], (int)aw[4], (int)aw[5], 0, 0};
    const v8i a1 = {(int)aw[6], (int)aw[7], (int)aw[8], (int)aw[9], (int)aw[10], (int)aw[11], 0, 0};
    const v8i a2 = {(int)aw[12], (int)aw[13], (int)aw[14], (int)aw[15], (int)aw[16], (int)aw[17], 0, 0};
    const int sw = (int)aw[18];
    const int s0 = sw & 0xff, s1 = (sw >> 8) & 0xff, s2 = (sw >> 16) & 0xff;
    v8i b[NCB];
    int bsc[NCB];
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      b[j] = (v8i){(int)(st.bc[j].x & keep), (int)(st.bc[j].y & keep), (int)(st.bc[j].z & keep),
                   (int)(st.bc[j].w & keep), 0, 0, 0, 0};
      bsc[j] = (int)(((uint32_t)st.bs[j] & keep) | (127u & ~keep));
    }
    // term-major order: consecutive MFMAs use different accumulators
#pragma unroll
    for (int j = 0; j < NCB; ++j)
      acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b[j], acc[mb][j], 2, 4, 0, s0, 0, bsc[j]);
    if constexpr (TERMS >= 2) {
#pragma unroll
      for (int j = 0; j < NCB; ++j)
        acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b[j], acc[mb][j], 2, 4, 0, s1, 0, bsc[j]);
    }
    if constexpr (TERMS == 3) {
#pragma unroll
      for (int j = 0; j < NCB; ++j)
        acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a2, b[j], acc[mb][j], 2, 4, 0, s2, 0, bsc[j]);
    }
  }
}

__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Maximum over the 16 lanes of a DPP row (lanes 16g .. 16g+15): rotations
// by 8, 4, 2, 1 within the row leave every lane holding the row maximum.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));
  return v;
}

// MX6x3 split of one 32-column block of h held as two values per lane by
// the 16 lanes of a DPP row (columns r and 16 + r): writes the row's codes
// to LDS s_codes_row[3][32] and returns the packed scale word.
__device__ __forceinline__ uint32_t split_h_row(float h0, float h1, int r, uint8_t (*s_codes_row)[32]) {
  uint32_t scw = 0;
#pragma unroll
  for (int t = 0; t < 3; ++t) {
    float amax = fmaxf(fabsf(h0), fabsf(h1));
    if (h0 != h0 || h1 != h1) amax = __builtin_inff();
    amax = row16_max(amax);
    const int se = mx6_scale_exp(amax);
    scw |= (uint32_t)se << (8 * t);
    uint32_t k0 = 0, k1 = 0;
    if (se != 255) {
      const int kk = se - 127;
      const float ih = exp2i(-(kk >> 1)), il = exp2i(-(kk - (kk >> 1)));
      const float sh = exp2i(kk >> 1), sl = exp2i(kk - (kk >> 1));
      float q0, q1;
      k0 = e2m3_round((h0 * ih) * il, q0);
      k1 = e2m3_round((h1 * ih) * il, q1);
      h0 -= (q0 * sh) * sl;
      h1 -= (q1 * sh) * sl;
    }
    s_codes_row[t][r] = (uint8_t)k0;
    s_codes_row[t][16 + r] = (uint8_t)k1;
  }
  return scw;
}

// ---------------------------------------------------------------------------
// Decode kernel: tiles of at most 16 rows, so the kernel is bound by the
// weight stream.  Work items are (tile, 64-row weight span) pairs (gate/up:
// 32 gate + the matching 32 up rows; down: 64 output rows), numbered
// tile-major, one per workgroup; four workgroups share a CU, so one's
// start and epilogue overlap the others' streams.  (Measured slower: a
// persistent variant that walks several items and overlaps each epilogue
// with the next item's first copies -- it needs more registers per lane --
// and a variant that loads the codes straight into the MFMA operand
// registers, each wave walking its own K steps with two in flight, about
// 1.5 us per 20b gate/up launch.)  An item walks K in phases of DEC_KPH
// blocks.  Wave w
// copies the phase's code and scale segments of column block w (16
// consecutive weight rows) from HBM straight to LDS with buffer_load ... lds
// -- no register staging, and every instruction reads 1 KB of
// lane-consecutive addresses, so whole cache lines are fetched (the scale
// bytes land one per LDS dword, the layout of byte loads to LDS).  Within a
// row the blocks of a phase are stored XOR-swizzled (logical block b of row
// j at slot b ^ (j & 15)), so the MFMA operand reads -- 16 rows x one block
// per lane group -- hit distinct LDS banks.  A rows come from the MX6x3
// buffer through a buffer resource: lanes of rows past the tile read at an
// offset beyond the resource, which returns zero without touching memory.
// The four waves split each phase's blocks; the epilogue sums their
// partials in a fixed order.
typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte copy to LDS, in a plain (non-template) function: the compiler's
// host pass cannot check this size against its own target, which it would
// have to do for a call with template-dependent arguments
__device__ __forceinline__ void lds_copy16(__amdgpu_buffer_rsrc_t rsrc, lds_void_t* dst, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, dst, 16, (int)voffset, 0, 0, 0);
}

constexpr int DEC_KPH = 16;                // K blocks per phase
constexpr int DEC_NW = 4;                  // waves per workgroup
constexpr int DEC_Q = DEC_KPH / 4;         // copy instructions per wave per phase (codes; same for scales)
constexpr int DEC_WB = DEC_KPH / DEC_NW;   // blocks per wave per phase (4 = one chunk)
// Scale bytes go to LDS with 2-byte copies when a weight row's scale bytes
// start 2-byte aligned (K/32 even): lane L's two bytes land in LDS dword L,
// so a wave moves its 16 rows x 16 blocks in two instructions and a phase
// buffer holds 8 dwords per weight row; otherwise with 1-byte copies (four
// instructions, 16 dwords per row).  The smaller buffers let four
// workgroups share a CU.
template <bool U16>
struct DecCfg {
  static constexpr int SQ = U16 ? 2 : DEC_Q;                // scale copy instructions per wave per phase
  static constexpr int SROW = U16 ? DEC_KPH / 2 : DEC_KPH;  // scale dwords per weight row
  static constexpr int VM = DEC_Q + SQ + 5;                 // vector-memory instructions per wave per phase
  static constexpr int WG_PER_CU = U16 ? 4 : 3;             // resident workgroups per CU
};
static_assert(DEC_WB == 4, "one 4-block chunk per wave per phase");

// Everything the decode kernel needs to know about one work item.
struct DecItem {
  int e, m0, rows, row_base, col0;
  int pair;                         // lane r's row: its (token, slot) pair (row r < rows)
  int ok_mask;                      // bit j: column block j lies inside the output
  __amdgpu_buffer_rsrc_t crsrc;     // this wave's 16 weight rows: codes
  __amdgpu_buffer_rsrc_t srsrc;     //   and scales
  int a_off[2];                     // this lane's A row offsets (rows r, r + 16), or past the A resource
  int rs;                           // weight rows between consecutive columns of a block (1, or 2 interleaved)
  int row0;                         // packed layout: this wave's first weight row within the expert
  float bias[4];                    // this lane's epilogue bias values (gate/up: gate and up of
                                    // columns col0 + r and col0 + 16 + r; down: column col0 + 16j + r)
};

// The tile list, counts, offsets and row lists were written by an earlier
// launch and are only read here, so they are read as constant memory:
// scalar loads of uniform values (the expert's 16 row-list entries of the
// tile too, then picked per lane by a select ladder).
typedef __attribute__((address_space(4))) const int cint_t;

// The head of an item: what its weight copies need (the tile's expert e and
// first row m0, already loaded, and the item's column span), so that the
// first copies go out before the row list is read.
template <bool GATEUP, bool PACKED = false>
__device__ __forceinline__ void dec_item_head(const GemmParams& p, int e, int m0, int span, int wave, DecItem& it) {
  const int K = p.K, N = p.N, I = p.I, nblk = K >> 5;
  it.e = e;
  it.m0 = m0;
  int ok = 0;
  if (GATEUP) {
    it.col0 = span * 32;
    ok = (it.col0 < I ? 0x5 : 0) | (it.col0 + 16 < I ? 0xA : 0);
  } else {
    it.col0 = span * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j) ok |= (it.col0 + 16 * j < N) ? (1 << j) : 0;
  }
  it.ok_mask = ok;
  // first weight row of this wave's column block (a missing block copies
  // block 0); its 16 rows are consecutive weight rows
  const int cbv = ((ok >> wave) & 1) ? wave : 0;
  const int n = GATEUP ? gu_row(it.col0 + 16 * (cbv & 1), cbv >= 2, I, p.alt) : it.col0 + 16 * cbv;
  it.rs = (GATEUP && p.alt) ? 2 : 1;
  const size_t my_row = (size_t)e * N + n;
  it.row0 = n;
  if constexpr (PACKED) {
    // the pair of my_row onwards (codes), the expert's chunk-major scales
    // onwards; both end at the end of their arrays
    const size_t pair = my_row >> 1, nchk = (size_t)((nblk + 3) >> 2);
    it.crsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.b_codes + pair * (size_t)K), 0,
                                                 (int)(((size_t)p.E * (N >> 1) - pair) * (size_t)K), 0x00020000);
    it.srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.b_scales + (size_t)e * nchk * N * 4), 0,
                                                 (int)((size_t)(p.E - e) * nchk * N * 4), 0x00020000);
  } else {
    // resources end at the end of the arrays, so that copies past the last
    // row return zeros instead of reading past the allocation
    const size_t rows_left = (size_t)p.E * N - my_row;
    it.crsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.b_codes + my_row * (size_t)(K >> 1)), 0,
                                                 (int)(rows_left * (size_t)(K >> 1)), 0x00020000);
    it.srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(p.b_scales + my_row * (size_t)nblk), 0,
                                                 (int)(rows_left * (size_t)nblk), 0x00020000);
  }
}

// The tail of an item: its rows (count, place in the grouped order, the
// row list) and A offsets, and the epilogue's bias.
template <bool GATEUP, int MB>
__device__ __forceinline__ void dec_item_tail(const GemmParams& p, int r, DecItem& it) {
  const int N = p.N, I = p.I, nblk = p.K >> 5;
  const int e = it.e, m0 = it.m0;
  it.rows = min(16 * MB, ((cint_t*)p.counts)[e] - m0);
  it.row_base = ((cint_t*)p.offsets)[e] + m0;
  int arow[2] = {it.row_base + r, it.row_base + 16 + r};
  if (GATEUP) {
    // entries past the expert's T read on into the next expert's list or
    // the workspace region after the lists; they are never used
    cint_t* erow = (cint_t*)p.expert_rows + (size_t)e * p.T + m0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = erow[16 * mb + i];
      int x = v[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) x = r == i ? v[i] : x;
      if (mb == 0) it.pair = x;
      arow[mb] = x / p.k;
    }
  } else {
    // (entries past the expert's rows are read but never used, as above)
    it.pair = p.expert_rows[(size_t)e * p.T + m0 + r];
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
    it.a_off[mb] = (mb < MB && 16 * mb + r < it.rows) ? arow[mb] * mx6_row_bytes(nblk) : 0x7ffffff0;
  // the epilogue's bias, loaded now so that its latency hides under the
  // weight stream (columns past the output read the last column, never
  // stored)
  const float* bias = p.bias + (size_t)e * N;
  if (GATEUP) {
    const int c0 = min(it.col0 + r, I - 1), c1 = min(it.col0 + 16 + r, I - 1);
    it.bias[0] = bias[gu_row(c0, 0, I, p.alt)];
    it.bias[1] = bias[gu_row(c0, 1, I, p.alt)];
    it.bias[2] = bias[gu_row(c1, 0, I, p.alt)];
    it.bias[3] = bias[gu_row(c1, 1, I, p.alt)];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) it.bias[j] = bias[min(it.col0 + 16 * j + r, N - 1)];
  }
}

// An item whose copies all fall outside their resources: they return zeros
// without touching memory (issued after the last real phase so that every
// step has the same shape).
__device__ __forceinline__ void dec_null_item(const GemmParams& p, DecItem& it) {
  it.e = 0; it.m0 = 0; it.pair = 0; it.rows = 0; it.row_base = 0; it.col0 = 0; it.ok_mask = 0;
  it.crsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.b_codes, 0, 0, 0x00020000);
  it.srsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.b_scales, 0, 0, 0x00020000);
  it.a_off[0] = it.a_off[1] = 0x7ffffff0;
  it.rs = 1;
  it.row0 = 0;
  it.bias[0] = it.bias[1] = it.bias[2] = it.bias[3] = 0.f;
}

// MB = 2: 32-row tiles (two A row blocks per lane), for batches of up to
// 32 rows per expert, so that an expert's weights are read once.
// PACKED (with U16): the weights in the packed layout of moe_pack_weights;
// the copies put the same bytes into the same LDS places.
template <bool GATEUP, int NPH, bool U16, int TERMS, int MB, bool PACKED = false>
__global__ __launch_bounds__(DEC_NW * 64, MB == 1 ? DecCfg<U16>::WG_PER_CU : 3) void expert_gemm_decode(GemmParams p,
                                                                                                     int spans) {
  static_assert(!PACKED || U16, "the packed layout has K/32 even");
  using Cfg = DecCfg<U16>;
  // vector-memory instructions per wave per phase (one term loads two
  // fewer A pieces per row block, two terms one fewer)
  // the packed layout's chunk-major scales go to LDS with one 4-byte copy
  // per wave and phase (four dwords per weight row), the row-major scales
  // with 2-byte (U16) or 1-byte copies
  constexpr int SROW = PACKED ? 4 : Cfg::SROW;
  constexpr int SQ = PACKED ? 1 : Cfg::SQ;
  constexpr int VM = DEC_Q + SQ + MB * (TERMS == 1 ? 3 : TERMS == 2 ? 4 : 5);
  constexpr int NCB = 4, NW = DEC_NW;
  // readfirstlane: the wave index is uniform, so the buffer resources and
  // LDS bases derived from it live in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the item's tile entry is read together with the tile count (the list
  // has room for every tile of the grid): one round trip for both
  const int item = blockIdx.x, tile = item / spans, span = item - tile * spans;
  const int n_tiles = *(cint_t*)p.n_tiles;
  const int te_e = ((cint_t*)p.tiles)[2 * tile], te_m0 = ((cint_t*)p.tiles)[2 * tile + 1];
  asm volatile("" ::"s"(n_tiles), "s"(te_e), "s"(te_m0));
  if (item >= n_tiles * spans) return;
  const int K = p.K, N = p.N, I = p.I, nblk = K >> 5;
  const int g = lane >> 4, r = lane & 15;
  const int nph = (nblk + DEC_KPH - 1) / DEC_KPH;

  // two phase buffers: codes [64 rows][16 slots][16 B], scales one per dword
  __shared__ __align__(16) uint8_t s_code[2][64 * DEC_KPH * 16];
  __shared__ __align__(16) uint32_t s_scl[2][64 * SROW];
  __shared__ uint8_t s_codes[16][3][32];
  __shared__ uint32_t s_sc[16];

  // A rows through a buffer resource over the whole MX6x3 buffer (the
  // library keeps it below 2 GiB); a lane's offset selects row and block
  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc((void*)p.a, 0, 0x7ffffff0, 0x00020000);

  // issue every load of phase ph of item `it`: this wave's column block
  // into LDS buffer `buf` (instruction q moves rows 4q .. 4q+3), this wave's
  // A block into av
  const int lane_id = lane;
  // The phase's own offset goes into the instructions' scalar offset (pb0
  // blocks: 16 B of codes, 1 B of scales, 80 B of A per block), so the lane
  // offsets are the same for every full phase and need no registers per
  // phase.  The bounds checks only ever rely on lane offsets: rows past an
  // item and the null item's copies have lane offsets at or past the
  // resource's end; every other access lies inside its row.
  // (with the phase count known, every phase but the last is full: its
  // offsets are then the same in every phase)
  auto issue_b = [&](const DecItem& it, int ph, int buf) {
    // the lane offsets are recomputed at every issue (a few instructions)
    // rather than held in registers across the item loop
    int lane = lane_id;
    asm volatile("" : "+v"(lane));
    const int sub = lane / DEC_KPH, slot = lane % DEC_KPH;
    const int pb0 = ph * DEC_KPH, npb = (NPH > 0 && ph < NPH - 1) ? DEC_KPH : min(DEC_KPH, nblk - pb0);
#pragma unroll
    for (int q = 0; q < DEC_Q; ++q) {
      const int rr = 4 * q + sub;                  // row within the column block
      const int b = min(slot ^ rr, npb - 1);       // logical block stored at `slot`
      const int row_off = (wave * 16 + 4 * q) * DEC_KPH;
      if constexpr (PACKED) {
        // weight row row0 + rr * rs sits in pair (row0 + rr * rs) / 2 (from
        // the resource's pair), its chunk c at 128 c + half * w_c there; the
        // phase's 4 chunks of a pair are 512 bytes (the scalar offset)
        const int wr = (it.row0 & 1) + rr * it.rs, bb = pb0 + b, c = bb >> 2;
        const int w = 4 * c + 4 <= nblk ? 64 : 16 * (nblk - 4 * c);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(it.crsrc, (lds_void_t*)(s_code[buf] + row_off * 16), 16,
                                                 (wr >> 1) * K + 128 * (b >> 2) + (wr & 1) * w + 16 * (b & 3),
                                                 pb0 * 32, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(it.crsrc, (lds_void_t*)(s_code[buf] + row_off * 16), 16,
                                                 rr * it.rs * (K >> 1) + b * 16, pb0 * 16, 0, 0);
      }
      if constexpr (!U16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(it.srsrc, (lds_void_t*)(s_scl[buf] + row_off), 1,
                                                 rr * it.rs * nblk + min(slot, npb - 1), pb0, 0, 0);
    }
    if constexpr (PACKED) {
      // one 4-byte copy: lane L fills dword L of the wave's 16 rows x 4
      // dwords; row rr = L / 4 keeps chunk (L % 4) ^ ((rr >> 3) & 1) of the
      // phase (the scale bytes of its blocks 4c .. 4c+3, from chunk pb0 / 4
      // + c of the chunk-major scales, the chunk of pb0 in the scalar
      // offset) in slot L % 4, so that the reads of one chunk by 16 rows
      // hit 16 banks.  Chunks past K read on past the expert's scales (or
      // past the resource: zeros); their blocks are masked off.
      const int rr = lane >> 2;
      const int c = (lane & 3) ^ ((rr >> 3) & 1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(it.srsrc, (lds_void_t*)(s_scl[buf] + wave * 16 * SROW), 4,
                                               (c * N + it.row0 + rr * it.rs) * 4, pb0 * N, 0, 0);
    } else if constexpr (U16) {
      // instruction q moves rows 8q .. 8q+7; lane L holds the block pair
      // (L % 8) ^ ((row >> 2) & 3) of row 8q + L/8, so that the reads of 16
      // rows hit 16 banks; pairs past the phase read pair 0 (never used)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int rr = 8 * q + (lane >> 3);
        const int u = (lane & 7) ^ ((rr >> 2) & 3);
        const int uc = 2 * u < npb ? u : 0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(it.srsrc,
                                                 (lds_void_t*)(s_scl[buf] + (wave * 16 + 8 * q) * SROW), 2,
                                                 rr * it.rs * nblk + 2 * uc, pb0, 0, 0);
      }
    }
  };
  auto issue_a = [&](const DecItem& it, int ph, uint4 (&av)[MB][5]) {
    const int g = lane_id >> 4;
    const int pb0 = ph * DEC_KPH, npb = (NPH > 0 && ph < NPH - 1) ? DEC_KPH : min(DEC_KPH, nblk - pb0);
    // block pb0 + 4w + g of the phase (blocks past K read the last block;
    // their products are masked off); piece q of the lanes g = 0..3 is one
    // 64-byte line of the piece-interleaved row
    const int bl = min(wave * DEC_WB + g, npb - 1);
    const int aso = pb0 / 4 * MX6_GROUP_BYTES;  // pb0 is a multiple of 4 blocks
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int off = it.a_off[mb] < 0x7ffffff0 ? it.a_off[mb] + mx6_byte_offset(bl, 0) : 0x7ffffff0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q > TERMS && q < 4) {  // pieces 2 and 3 hold only the later terms' codes
          av[mb][q] = make_uint4(0u, 0u, 0u, 0u);
          continue;
        }
        const auto t4 = __builtin_amdgcn_raw_buffer_load_b128(arsrc, off + 64 * q, aso, 0);
        av[mb][q] = make_uint4(t4[0], t4[1], t4[2], t4[3]);
      }
      // bytes 64 .. 75: the last term's codes and the scale bytes (the
      // padding dword is not loaded: a register that a load in flight
      // writes must not be dead, or the compiler waits for the load before
      // reusing it)
      const auto t3 = __builtin_amdgcn_raw_buffer_load_b96(arsrc, off + 256, aso, 0);
      av[mb][4] = make_uint4(t3[0], t3[1], t3[2], 0u);
    }
  };
  auto issue = [&](const DecItem& it, int ph, int buf, uint4 (&av)[MB][5]) {
    issue_b(it, ph, buf);
    issue_a(it, ph, av);
  };

  v4f acc[MB][NCB];
  auto consume = [&](int ph, int buf, const uint4 (&av)[MB][5]) {
    const int npb = (NPH > 0 && ph < NPH - 1) ? DEC_KPH : min(DEC_KPH, nblk - ph * DEC_KPH);
    const int bl = wave * DEC_WB + g;  // logical block within the phase
    Stage<MB, NCB> st;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 5; ++q) st.a[mb][q] = av[mb][q];
    // The LDS reads are written as one asm block that waits for its own
    // results: the compiler cannot tell the two phase buffers apart, and
    // would otherwise wait for every copy in flight (the next phase's too)
    // before reading.  The barriers and explicit vmcnt waits order them.
    const uint32_t cb_addr = (uint32_t)(uintptr_t)(s_code[buf]) + (uint32_t)((r * DEC_KPH + (bl ^ r)) * 16);
    const uint32_t sb_addr =
        (uint32_t)(uintptr_t)(s_scl[buf]) +
        (uint32_t)((PACKED ? r * SROW + ((bl >> 2) ^ ((r >> 3) & 1))
                    : U16  ? r * SROW + ((bl >> 1) ^ ((r >> 2) & 3))
                           : r * DEC_KPH + bl) *
                   4);
    v4u b0, b1, b2, b3;
    uint32_t s0, s1, s2, s3;
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:%10\n\t"
        "ds_read_b128 %2, %8 offset:%11\n\t"
        "ds_read_b128 %3, %8 offset:%12\n\t"
        "ds_read_b32 %4, %9\n\t"
        "ds_read_b32 %5, %9 offset:%13\n\t"
        "ds_read_b32 %6, %9 offset:%14\n\t"
        "ds_read_b32 %7, %9 offset:%15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
        : "v"(cb_addr), "v"(sb_addr), "i"(16 * DEC_KPH * 16), "i"(32 * DEC_KPH * 16), "i"(48 * DEC_KPH * 16),
          "i"(16 * SROW * 4), "i"(32 * SROW * 4), "i"(48 * SROW * 4));
    st.bc[0] = make_uint4(b0.x, b0.y, b0.z, b0.w);
    st.bc[1] = make_uint4(b1.x, b1.y, b1.z, b1.w);
    st.bc[2] = make_uint4(b2.x, b2.y, b2.z, b2.w);
    st.bc[3] = make_uint4(b3.x, b3.y, b3.z, b3.w);
    // byte of the block within its chunk (packed) or pair (U16)
    const int sh = PACKED ? 8 * (bl & 3) : U16 ? 8 * (bl & 1) : 0;
    st.bs[0] = (int)((s0 >> sh) & 0xffu);
    st.bs[1] = (int)((s1 >> sh) & 0xffu);
    st.bs[2] = (int)((s2 >> sh) & 0xffu);
    st.bs[3] = (int)((s3 >> sh) & 0xffu);
    mma_stage<MB, NCB, TERMS>(acc, st, keep_mask<MB, NCB>(bl < npb));
    // pin the MFMAs to this phase: unused until the epilogue, they could
    // otherwise be sunk past later code, holding every phase's operands
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      asm volatile("" : "+v"(acc[mb][0]), "+v"(acc[mb][1]), "+v"(acc[mb][2]), "+v"(acc[mb][3]));
  };

  // ---- epilogue of item `it`: wave w takes accumulator element w, i.e.
  // tile rows 4g + w, and sums the four waves' partials in a fixed order.
  // s_acc is the phase buffer consumed last (free until the next issue).
  // With two row blocks it runs once per block (tile rows 16 mb + 4g + w).
  auto epilogue = [&](const DecItem& it, float* s_acc, auto mbc) {
    constexpr int mb = decltype(mbc)::value;
#pragma unroll
    for (int j = 0; j < NCB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) s_acc[((wave * NCB + j) * 4 + q) * 64 + lane] = acc[mb][j][q];
    wait_lgkmcnt<0>();  // the partials are in LDS
    __builtin_amdgcn_s_barrier();
    float v[NCB];
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      float t = s_acc[((0 * NCB + j) * 4 + wave) * 64 + lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) t += s_acc[((w * NCB + j) * 4 + wave) * 64 + lane];
      v[j] = t;
    }
    const int lrow = 4 * g + wave, row = 16 * mb + lrow;  // tile row of this lane's values
    const int col0 = it.col0, rows = it.rows, row_base = it.row_base;
    if (!GATEUP) {
      const bool fold = MB == 1 && p.fold_cnt != nullptr;
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        if (!((it.ok_mask >> j) & 1)) continue;
        const int col = col0 + 16 * j + r;
        if (row < rows) {
          const size_t o = (size_t)(row_base + row) * N + col;
          // (with the fold, a device-coherent store: see below)
          if (fold)
            __hip_atomic_store(p.y + o, v[j] + it.bias[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            p.y[o] = v[j] + it.bias[j];
        }
      }
      if (!fold) return;
      // The combine, folded in: once every wave's rows have landed, one lane
      // per tile row counts its token in for this 64-column span; the
      // arrival that completes a token's k rows sums them for the span, in
      // slot order, exactly as the separate combine does (an fma per slot,
      // one rounding to bf16).  The router launch cleared the counters.
      //
      // Ordering across workgroups (the last arrival may run on another
      // XCD, whose L2 is not coherent with this one's): the rows are stored
      // with agent-scope atomic stores, which gfx950 writes through to the
      // device-coherent level, and every wave waits for its stores to
      // complete (vmcnt 0) before the workgroup barrier that precedes the
      // arrival, so the arrival is performed after the rows are visible at
      // that level; the last arrival reads them with agent-scope atomic
      // loads, which read from that level, issued after it has seen the
      // count.  An acquire-release arrival would order the same accesses in
      // the language's memory model, but on gfx950 it writes back the XCD's
      // whole L2 once per workgroup: 103 instead of 36.5 us for the 20b
      // decode down projection.
      // First the slots of the tile rows' tokens, one (row, slot) per thread
      // of the first two waves: where each sits in y (the gate/up launch
      // recorded it) and its weight, issued before the wait for the stores
      // so that the two round trips overlap.
      const int k = p.k, tok_r = it.pair / k;
      int fpos = 0;
      float fw = 0.f;
      if (tid < 128) {
        const int i = tid >> 3, j = tid & 7, ti = __shfl(tok_r, i);
        if (i < rows && j < k) {
          fpos = p.pair_row[ti * k + j];
          fw = p.topk_w[ti * k + j];
        }
      }
      wait_vmcnt<0>();  // this wave's rows are stored
      // (staged in the split's buffers, unused by the down projection)
      int* s_tok = (int*)s_sc;
      int* s_pos = (int*)&s_codes[0][0][0];
      float* s_w = (float*)s_pos + 128;
      if (tid < 128) {
        s_pos[tid] = fpos;
        s_w[tid] = fw;
      }
      __syncthreads();
      const int spans = (N + 63) >> 6, span = col0 >> 6;
      if (wave == 0 && lane < 16) {
        int t = -1;
        if (lane < rows &&
            __hip_atomic_fetch_add(p.fold_cnt + (size_t)tok_r * spans + span, 1, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT) == k - 1)
          t = tok_r;
        s_tok[lane] = t;
      }
      __syncthreads();
      // each wave sums tile rows wave, wave + 4, ... for the span's 64
      // columns, one per lane; every y load of the wave is issued before
      // the first sum
      static_assert(NW * 4 == 16, "four tile rows per wave");
      const int col = col0 + lane, colc = min(col, N - 1);
      int tq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = wave + NW * q;
        tq[q] = i < rows ? s_tok[i] : -1;
      }
      float yv[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (tq[q] >= 0 && j < k)
            yv[q][j] = __hip_atomic_load(p.y + (size_t)s_pos[(wave + NW * q) * 8 + j] * N + colc, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (tq[q] < 0 || col >= N) continue;
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j < k) acc = fmaf(s_w[(wave + NW * q) * 8 + j], yv[q][j], acc);
        const size_t o = (size_t)tq[q] * N + col;
        if (p.out_f32) p.out_f32[o] = acc;
        p.out[o] = f32_to_bf16(acc);
      }
      return;
    }
    // (columns past I are never stored)
    const float h0 = swiglu_act(v[0] + it.bias[0], v[2] + it.bias[1], p.clamp, p.alt);
    const float h1 = swiglu_act(v[1] + it.bias[2], v[3] + it.bias[3], p.clamp, p.alt);
    const uint32_t scw = split_h_row(h0, h1, r, s_codes[lrow]);
    if (r == 0) s_sc[lrow] = scw;
    lds_wave_sync();
    const int blk = col0 >> 5;
    if (lane < 12) {
      const int rw = 4 * (lane / 3) + wave, t = lane % 3;
      if (16 * mb + rw < rows) {
        uint32_t pk[6];
        pack6x32(s_codes[rw][t], pk);
        uint8_t* hrow = p.hq + (size_t)(row_base + 16 * mb + rw) * mx6_row_bytes(I >> 5);
        // 8-byte stores at multiples of 8 never straddle a 16-byte piece
        *(uint2*)(hrow + mx6_byte_offset(blk, 24 * t)) = make_uint2(pk[0], pk[1]);
        *(uint2*)(hrow + mx6_byte_offset(blk, 24 * t + 8)) = make_uint2(pk[2], pk[3]);
        *(uint2*)(hrow + mx6_byte_offset(blk, 24 * t + 16)) = make_uint2(pk[4], pk[5]);
      }
    } else if (lane < 16) {
      const int rw = 4 * (lane - 12) + wave;
      if (16 * mb + rw < rows) {
        uint8_t* hrow = p.hq + (size_t)(row_base + 16 * mb + rw) * mx6_row_bytes(I >> 5);
        *(uint2*)(hrow + mx6_byte_offset(blk, 72)) = make_uint2(s_sc[rw], 0u);
      }
    }
    lds_wave_sync();
  };

  // The phase loop.  Each step: issue the copies of the next phase (past the
  // last phase, of the null item, so that every step has the same shape),
  // wait for this wave's copies of the current phase (vmcnt counts in issue
  // order; the next phase's DEC_VM operations may stay in flight), publish
  // them with a bare s_barrier -- a __syncthreads() would make the compiler
  // drain every copy in flight -- and consume.  The second barrier keeps a
  // buffer from being refilled while another wave still reads it.  With the
  // phase count known at compile time (NPH > 0) the loop is unrolled, so the
  // A registers of consecutive phases are fixed and no copy of a load in
  // flight forces an early wait; the scheduling barrier keeps the consume's
  // register moves behind the wait.
  // The first phase's weight copies go out as soon as the expert is known;
  // the row list, the A offsets and the bias follow.
  DecItem cur, nul;
  dec_item_head<GATEUP, PACKED>(p, te_e, te_m0, span, wave, cur);
  issue_b(cur, 0, 0);
  dec_item_tail<GATEUP, MB>(p, r, cur);
  dec_null_item(p, nul);
  // for the down projection's folded combine: where each pair's row sits
  // (single row block only)
  if (GATEUP && MB == 1 && p.pair_row != nullptr && cur.col0 == 0 && wave == 0 && lane < cur.rows)
    p.pair_row[cur.pair] = cur.row_base + lane;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NCB; ++j) acc[mb][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  uint4 av0[MB][5], av1[MB][5];
  issue_a(cur, 0, av0);
  // step of phase ph: copies of phase ph + 1 of `cur`, or (last phase) of
  // phase 0 of `nit`
  auto step = [&](int ph, int buf, bool last, const DecItem& nit, const uint4 (&avc)[MB][5], uint4 (&avn)[MB][5]) {
    if (last)
      issue(nit, 0, buf ^ 1, avn);
    else
      issue(cur, ph + 1, buf ^ 1, avn);
    wait_vmcnt<VM>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    consume(ph, buf, avc);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // With the phase count known at compile time (NPH > 0) the loop is
  // unrolled, so the A registers of consecutive phases are fixed and no copy
  // of a load in flight forces an early wait.
  if constexpr (NPH > 0) {
    StaticFor<0, NPH>::run([&](auto pc) {
      constexpr int ph = decltype(pc)::value;
      if constexpr (ph % 2 == 0)
        step(ph, 0, ph == NPH - 1, nul, av0, av1);
      else
        step(ph, 1, ph == NPH - 1, nul, av1, av0);
    });
  } else {
    for (int ph = 0;;) {
      step(ph, 0, ph + 1 >= nph, nul, av0, av1);
      if (++ph >= nph) break;
      step(ph, 1, ph + 1 >= nph, nul, av1, av0);
      if (++ph >= nph) break;
    }
  }
  wait_vmcnt<0>();  // the null item's copies
  epilogue(cur, (float*)s_code[(nph - 1) & 1], std::integral_constant<int, 0>{});
  if constexpr (MB == 2) {
    __syncthreads();  // every wave has read its sums of the first row block
    epilogue(cur, (float*)s_code[(nph - 1) & 1], std::integral_constant<int, 1>{});
  }
}

// Prefill kernel: tiles of PF_MT = 64 rows x 256 output columns (gate/up:
// 128 gate + the matching 128 up columns).  A workgroup has four waves and
// two workgroups share a CU, so every SIMD runs two waves (a single wave per
// SIMD issues the block-scaled MFMAs at only about 60% of the pipe's rate)
// and one workgroup's start and epilogue overlap the other's K loop (a
// single 8-wave workgroup with 128 x 384 tiles measured slower).  Wave
// (wm, wn) owns rows 32wm .. 32wm+31 (two 16-row blocks) and column half wn
// (gate/up: 64 gate + 64 up columns, i.e. two whole MX blocks of h), eight
// 16-column blocks in all, so every B fragment read from LDS feeds six
// MFMAs.  K advances in
// chunks of four 32-element blocks.  Each wave loads its A fragments
// straight from global memory into registers, one chunk ahead.  The weight
// tile goes through two LDS buffers: its global loads for chunk c+1 are
// issued into registers before chunk c is consumed and written to the
// other buffer after chunk c's MFMAs have been issued, one barrier per
// chunk.  Inside a chunk, B fragments are read from LDS PF_BPRE column
// blocks ahead of their MFMAs.  B rows are stored with their four 16-byte
// pieces XOR-swizzled by (row >> 2) & 3, so the fragment reads are free of
// LDS bank conflicts.
//
// Work items (tile, column span) are numbered tile-major and dealt to the
// eight XCDs in contiguous ranges (workgroup i runs on XCD i mod 8), so the
// column spans of one tile -- which share its A rows -- and the tiles of
// one expert -- which share its weights -- meet in the same L2.
constexpr int PF_MT = 64;                   // rows per tile
constexpr int PF_NT = 256;                  // weight rows (output columns) per tile
constexpr int PF_NW = 4;                    // waves: 2 row halves x 2 column halves
constexpr int PF_NCB = 8;                   // 16-column blocks per wave
constexpr int PF_XCD = 8;                   // XCDs of the device
constexpr int PF_BPRE = 2;                  // B fragments read ahead of their MFMAs

// Prefill epilogues.  After the K loop the operand buffers are free; the
// gate/up epilogue stages each wave's results in its own part of them, 16
// rows at a time.
//
// Gate/up: h = clamped SwiGLU of (gate + b13, up + b13) is written to LDS as
// fp32 [16][16*HALF + 4], each 32-column block stored as its 16 even then
// its 16 odd columns; then one lane per (row, 32-column block) reads the
// block, splits it into its three E2M3 terms with the hardware conversions
// and stores the 80-byte MX6x3 block as its five 16-byte pieces.
template <int NCB>
__device__ __forceinline__ void pf_epilogue_gateup(const GemmParams& p, const v4f (&acc)[2][NCB],
                                                   const float (&bias)[NCB], int rows_w, int row_base_w, int col0,
                                                   int lane, uint8_t* scratch) {
  constexpr int HALF = NCB / 2;      // gate column blocks
  constexpr int HS = 16 * HALF + 4;  // row stride of h in floats
  constexpr int NB = HALF / 2;       // MX blocks of h per row
  static_assert(HALF % 2 == 0, "gate span is whole 32-column blocks");
  float* sh_h = (float*)scratch;
  const int g = lane >> 4, r = lane & 15, I = p.I;
  const int nvalid = min(NB, (I - col0) >> 5);
  const size_t rowbytes = (size_t)mx6_row_bytes(I >> 5);
  // the block this lane splits: row lane / NB, block lane % NB
  const int srow = lane / NB, sblk = lane - srow * NB;
  // column 16j + r of the wave's span lies in block j / 2 at position
  // 16 (j & 1) + r, stored at 16 * (r & 1) + 8 (j & 1) + r / 2
  const int cpos = 16 * (r & 1) + (r >> 1);
  const SwigluConsts sk = swiglu_consts(p.clamp, p.alt);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (16 * mb >= rows_w) break;
#pragma unroll
    for (int j = 0; j < HALF; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        sh_h[(4 * g + q) * HS + 32 * (j >> 1) + 8 * (j & 1) + cpos] =
            clamped_swiglu(acc[mb][j][q] + bias[j], acc[mb][HALF + j][q] + bias[HALF + j], p.clamp, sk);
    lds_wave_sync();
    if (srow < 16) {
      const float* src = sh_h + srow * HS + 32 * sblk;
      v16f ve, vo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4f e4 = *(const v4f*)(src + 4 * i), o4 = *(const v4f*)(src + 16 + 4 * i);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ve[4 * i + u] = e4[u];
          vo[4 * i + u] = o4[u];
        }
      }
      uint32_t codes[18], scw;
      mx6x3_split_lane(ve, vo, codes, scw);
      if (16 * mb + srow < rows_w && sblk < nvalid) {
        // bytes 16q .. 16q+15 of the block go to piece q of its group
        uint8_t* dst = p.hq + (size_t)(row_base_w + 16 * mb + srow) * rowbytes;
        const int blk = (col0 >> 5) + sblk;
#pragma unroll
        for (int q = 0; q < 5; ++q) {
          const v4u piece = q < 4 ? (v4u){codes[4 * q], codes[4 * q + 1], codes[4 * q + 2], codes[4 * q + 3]}
                                  : (v4u){codes[16], codes[17], scw, 0u};
          *(v4u*)(dst + mx6_byte_offset(blk, 16 * q)) = piece;
        }
      }
    }
    lds_wave_sync();
  }
}

// Down: y = acc + b2 (fp32), stored straight from the accumulators: lane
// (g, r) holds rows 4g .. 4g+3 of each 16-row block in column r of each
// 16-column block, so the 16 lanes of a row group store 64 consecutive bytes
// of a row per column block (measured 1-3% faster than staging the rows
// through LDS and storing float4 pieces, and it needs no LDS).
template <int NCB>
__device__ __forceinline__ void pf_epilogue_down(const GemmParams& p, const v4f (&acc)[2][NCB],
                                                 const float (&bias)[NCB], int rows_w, int row_base_w, int col0,
                                                 int lane, uint8_t* /*scratch*/) {
  const int g = lane >> 4, r = lane & 15, N = p.N;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    if (16 * mb >= rows_w) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rw = 16 * mb + 4 * g + q;
      if (rw >= rows_w) continue;
      float* yr = p.y + (size_t)(row_base_w + rw) * N;
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        const int col = col0 + 16 * j + r;
        if (col < N) yr[col] = acc[mb][j][q] + bias[j];
      }
    }
  }
}

struct PfShared {
  uint8_t b[2][PF_NT * 64];
  uint8_t bs[2][PF_NT * 4];
};
// per-wave epilogue scratch: the gate/up staging (16 x (64 + 4) floats);
// the weight buffers share the same bytes (the epilogue starts after the
// loop's last barrier)
constexpr int PF_EPI_BYTES = 16 * (8 * PF_NCB + 4) * 4;
constexpr int PF_SMEM = (int)sizeof(PfShared) > PF_NW * PF_EPI_BYTES ? (int)sizeof(PfShared) : PF_NW * PF_EPI_BYTES;

template <bool GATEUP, int TERMS>
__global__ __launch_bounds__(PF_NW * 64, 2) void expert_gemm_prefill(GemmParams p, int spans) {
  constexpr int MB = 2, NCB = PF_NCB;
  constexpr int B_PIECES = PF_NT * 4 / (PF_NW * 64);  // 16-B weight pieces per thread per chunk
  static_assert(PF_NT * 4 % (PF_NW * 64) == 0, "even staging split");
  __shared__ __align__(16) uint8_t smem[PF_SMEM];
  PfShared& sh = *reinterpret_cast<PfShared*>(smem);

  // ---- work item ----
  const int total = *p.n_tiles * spans;
  const int per = (total + PF_XCD - 1) / PF_XCD;
  const int lin = blockIdx.x;
  const int item = (lin % PF_XCD) * per + lin / PF_XCD;
  if (lin / PF_XCD >= per || item >= total) return;
  const int tile = item / spans, span = item - tile * spans;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int rows = min(PF_MT, p.counts[e] - m0);
  const int row_base = p.offsets[e] + m0;
  const int K = p.K, N = p.N, I = p.I, nblk = K >> 5;
  const int g = lane >> 4, r = lane & 15;

  // tile columns: gate/up -- gate columns span*128 .. +127 (LDS rows 0..127)
  // and the same up columns (LDS rows 128..255); down -- span*256 .. +255
  const int tcol0 = GATEUP ? span * (PF_NT / 2) : span * PF_NT;
  // LDS row of the wave's column block j
  auto lds_row = [&](int j) -> int {
    if (GATEUP) return (j < NCB / 2 ? 0 : PF_NT / 2) + wn * (8 * NCB) + 16 * (j % (NCB / 2));
    return wn * (16 * NCB) + 16 * j;
  };

  // the tile's biases (by LDS row), loaded now so that they arrive during
  // the K loop; columns past the end are never stored
  const int wcol0 = GATEUP ? tcol0 + wn * (8 * NCB) : tcol0 + wn * (16 * NCB);
  __shared__ float s_bias[PF_NT];
  for (int n = tid; n < PF_NT; n += PF_NW * 64) {
    if (GATEUP) {
      const int c = min(tcol0 + (n % (PF_NT / 2)), I - 1);
      s_bias[n] = p.bias[(size_t)e * N + gu_row(c, n >= PF_NT / 2, I, p.alt)];
    } else {
      s_bias[n] = p.bias[(size_t)e * N + min(tcol0 + n, N - 1)];
    }
  }

  // ---- operand addressing: buffer resources over the whole A, code and
  // scale arrays (their sizes fit 32 bits; the launcher checks); each
  // lane's offsets are fixed over K and the chunk advance is a uniform
  // scalar offset.  Lanes past the end of K read the next row or past the
  // array (zero), and are masked off in the MFMAs.
  const uint32_t a_rowbytes = (uint32_t)mx6_row_bytes(nblk);
  const uint32_t a_rows_total = GATEUP ? (uint32_t)p.T : (uint32_t)(p.T * p.k);
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.a, 0, (int)(a_rows_total * a_rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.b_codes, 0, (int)((uint32_t)p.E * (uint32_t)N * (uint32_t)(K >> 1)), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.b_scales, 0, (int)((uint32_t)p.E * (uint32_t)N * (uint32_t)nblk), 0x00020000);
  // A: tile rows 32wm + 16mb + r (rows past the tile read tile row 0), block g of the chunk
  uint32_t a_off[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = 32 * wm + 16 * mb + r;
    const int m = row < rows ? row : 0;
    a_off[mb] = (GATEUP ? (uint32_t)(p.expert_rows[(size_t)e * p.T + m0 + m] / p.k) : (uint32_t)(row_base + m)) *
                    a_rowbytes + (uint32_t)g * 16u;
  }
  // weight piece q of this thread: LDS row n = tid/4 + 128q, 16-byte piece
  // tid % 4 of each chunk; columns past the end read the span's first block
  const int bpiece = tid & 3;
  uint32_t b_off[B_PIECES], s_off[B_PIECES];
  StaticFor<0, B_PIECES>::run([&](auto ic) {
    constexpr int q = decltype(ic)::value;
    const int n = (tid >> 2) + (PF_NW * 16) * q;
    int row;
    if (GATEUP) {
      const int c = tcol0 + (n % (PF_NT / 2));
      row = gu_row(c < I ? c : tcol0 + (n & 15), n >= PF_NT / 2, I, p.alt);
    } else {
      const int c = tcol0 + n;
      row = c < N ? c : tcol0 + (n & 15);
    }
    const uint32_t brow = (uint32_t)e * (uint32_t)N + (uint32_t)row;
    b_off[q] = brow * (uint32_t)(K >> 1) + (uint32_t)bpiece * 16u;
    s_off[q] = brow * (uint32_t)nblk + (uint32_t)bpiece;
  });

  // (one term loads pieces 0, 1 and 4 only: the first term's codes and the
  // scale bytes; two terms pieces 0, 1, 2 and 4)
  auto load_a = [&](int c, v4u (&av)[MB][5]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        if (q > TERMS && q < 4) {
          av[mb][q] = (v4u){0u, 0u, 0u, 0u};
          continue;
        }
        av[mb][q] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(arsrc, a_off[mb] + 64 * q,
                                                                                  c * MX6_GROUP_BYTES, 0));
      }
  };
  v4u rb[B_PIECES];
  uint32_t rs[B_PIECES];
  auto stage_load = [&](int c) {
    StaticFor<0, B_PIECES>::run([&](auto ic) {
      constexpr int q = decltype(ic)::value;
      rb[q] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(crsrc, b_off[q], c * 64, 0));
      rs[q] = __builtin_amdgcn_raw_buffer_load_b8(srsrc, s_off[q], c * 4, 0);
    });
  };
  // scale of (LDS row n, block g): LDS row n is column block j of column
  // half h (lds_row(j) of wave column h, row r); its byte sits at
  // (((h * NCB/4 + j/4) * 4 + g) * 16 + r) * 4 + j % 4, so one dword read
  // gives a lane the scales of four of its column blocks
  auto stage_store = [&](int buf) {
    StaticFor<0, B_PIECES>::run([&](auto ic) {
      constexpr int q = decltype(ic)::value;
      const int n = (tid >> 2) + (PF_NW * 16) * q;
      *(v4u*)(sh.b[buf] + n * 64 + ((bpiece ^ ((n >> 2) & 3)) * 16)) = rb[q];
      int h, j;
      if (GATEUP) {
        const int part = n >= PF_NT / 2, rem = n - part * (PF_NT / 2);
        h = rem / (8 * NCB);
        j = part * (NCB / 2) + (rem - h * (8 * NCB)) / 16;
      } else {
        h = n / (16 * NCB);
        j = (n - h * (16 * NCB)) / 16;
      }
      sh.bs[buf][(((h * (NCB / 4) + (j >> 2)) * 4 + bpiece) * 16 + (n & 15)) * 4 + (j & 3)] = (uint8_t)rs[q];
    });
  };

  v4f acc[MB][NCB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NCB; ++j) acc[mb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // One chunk: A fragments are taken out of the load registers, which are
  // refilled at once with the next chunk (as are the weight staging
  // registers); then the B fragments are read from LDS PF_BPRE column blocks
  // ahead of their MFMAs.  Lanes whose K block lies past the end of K
  // contribute zero codes with unit scales on both operands.  The body is
  // one basic block (the last iteration reloads the last chunk), so the
  // scheduling barriers keep the LDS stores behind the MFMAs and the global
  // loads' latency behind both.
  const int nchunk = (nblk + 3) >> 2;
  v4u av[MB][5];
  load_a(0, av);
  stage_load(0);
  stage_store(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int buf = c & 1;
    const uint32_t keep = (4 * c + g) < nblk ? 0xffffffffu : 0u;
    v8i a[MB][3];
    int as[MB][3];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      uint32_t w[20];
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        w[4 * q] = av[mb][q].x & keep; w[4 * q + 1] = av[mb][q].y & keep;
        w[4 * q + 2] = av[mb][q].z & keep; w[4 * q + 3] = av[mb][q].w & keep;
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        a[mb][t] = (v8i){(int)w[6 * t], (int)w[6 * t + 1], (int)w[6 * t + 2], (int)w[6 * t + 3], (int)w[6 * t + 4],
                         (int)w[6 * t + 5], 0, 0};
        as[mb][t] = (int)(((w[18] >> (8 * t)) & 0xffu) | (127u & ~keep));
      }
    }
    const int cn = min(c + 1, nchunk - 1);
    load_a(cn, av);
    stage_load(cn);
    __builtin_amdgcn_sched_barrier(0);
    // the wave's column blocks form groups of four consecutive LDS row
    // blocks, one scale dword each
    uint32_t bsw[NCB / 4];
#pragma unroll
    for (int h = 0; h < NCB / 4; ++h)
      bsw[h] = *(const uint32_t*)(sh.bs[buf] + (((wn * (NCB / 4) + h) * 4 + g) * 16 + r) * 4);
    v4u bq[PF_BPRE + 1];
    auto read_b = [&](int j) {
      const int n = lds_row(j) + r;
      bq[j % (PF_BPRE + 1)] = *(const v4u*)(sh.b[buf] + n * 64 + ((g ^ ((n >> 2) & 3)) * 16));
    };
    StaticFor<0, PF_BPRE>::run([&](auto jc) { read_b(decltype(jc)::value); });
    StaticFor<0, NCB>::run([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (j + PF_BPRE < NCB) read_b(j + PF_BPRE);
      const v4u b4 = bq[j % (PF_BPRE + 1)];
      const uint32_t braw = (bsw[j >> 2] >> (8 * (j & 3))) & 0xffu;
      const int bsc = (int)((braw & keep) | (127u & ~keep));
      const v8i b = {(int)(b4.x & keep), (int)(b4.y & keep), (int)(b4.z & keep), (int)(b4.w & keep), 0, 0, 0, 0};
      // the two row blocks alternate, so consecutive MFMAs never depend on
      // each other
#pragma unroll
      for (int t = 0; t < TERMS; ++t)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[mb][t], b, acc[mb][j], 2, 4, 0, as[mb][t],
                                                                        0, bsc);
      __builtin_amdgcn_sched_barrier(0);
    });
    stage_store((c + 1) & 1);
    __syncthreads();
  }

  // the loop's last barrier has passed: the weight buffers are free
  float bias[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) bias[j] = s_bias[lds_row(j) + r];
  const int rows_w = rows - 32 * wm;
  const int row_base_w = row_base + 32 * wm;
  uint8_t* scratch = smem + wave * PF_EPI_BYTES;
  if (GATEUP)
    pf_epilogue_gateup<NCB>(p, acc, bias, rows_w, row_base_w, wcol0, lane, scratch);
  else
    pf_epilogue_down<NCB>(p, acc, bias, rows_w, row_base_w, wcol0, lane, scratch);
}

// The prefill kernel addresses operands with 32-bit byte offsets.
// Wide prefill kernel: tiles of MT = 128 or 64 rows x PW_NT = 512 weight
// rows (gate/up: 256 gate + the matching 256 up columns), eight waves, one
// workgroup per CU.  Each wave owns 32 tile rows (two 16-row blocks) and
// 512 / WN weight rows (gate/up: half gate, half the matching up rows):
//   MT = 128: 4 x 2 waves, 16 column blocks per wave, so each A fragment
//     feeds 48 MFMAs and each B fragment 6.  With the three-term A operand
//     (80 bytes per 32 elements) the operands of a 64 x 256 tile need about
//     as many bytes per MFMA as a CU's L1 can deliver; this tile moves half
//     as many.
//   MT = 64: 2 x 4 waves, 8 column blocks per wave, for experts of fewer
//     than 64 rows (many experts and few tokens each: an expert's weights
//     are then read once, and HBM, not the MFMAs, bounds the kernel).  The
//     smaller A tile leaves room for three weight stages, so each CU keeps
//     two chunks of weights in flight instead of one.
//
// Both operands reach LDS with buffer_load ... lds (no register staging):
// per 4-block K chunk the A tile is MT rows x 320 bytes (one piece-
// interleaved group per row) and the weight tile 512 rows x 64 bytes of
// codes plus their scale bytes (2-byte copies, one per LDS dword).  Each
// copy instruction fills 1 KB (256 B for scales) of consecutive LDS, and
// the lane -> source mapping places the pieces XOR-swizzled (A: piece s of
// row m at slot s ^ ((m >> 1) & 3); B: piece g of row n at g ^ ((n >> 2) &
// 3)), so the fragment reads are free of bank conflicts.  A ring of two A
// stages and a ring of SB weight stages: after the barrier that opens
// chunk c, waves 4..7 issue the copies of A for chunk c+1 and of the
// weights for chunk c+SB-1, and each of them waits (vmcnt, in issue order)
// for its copies of chunk c before that barrier.  The LDS reads are asm blocks that
// wait for their own results, so the compiler never waits for the copies
// in flight.  Offsets include the chunk (no scalar offset): weight blocks
// past K are clamped to the row's last block, A rows past the tile read
// past the A resource (zeros, no traffic).
constexpr int PW_NT = 512;
constexpr int PW_NW = 8;
constexpr int PW_B_BYTES = PW_NT * 64;                // 32768
constexpr int PW_S_BYTES = PW_NT * 2 * 4;             // 4096
constexpr int PW_B_STAGE = PW_B_BYTES + PW_S_BYTES;
constexpr int PW_B_COPIES = PW_B_BYTES / 1024 / PW_NW;  // 4 per wave
constexpr int PW_S_COPIES = PW_NT * 2 / 64 / PW_NW;     // 2 per wave
static_assert(PW_B_COPIES == 4 && PW_S_COPIES == 2, "copy split");

template <int MT>
struct PwCfg {
  static_assert(MT == 128 || MT == 64, "128- or 64-row tiles");
  static constexpr int WN = MT == 128 ? 2 : 4;         // waves across the weight rows
  static constexpr int WM = PW_NW / WN;                // waves down the tile rows, 32 rows each
  static constexpr int NCB = PW_NT / 16 / WN;          // column blocks per wave
  static constexpr int A_BYTES = MT * MX6_GROUP_BYTES;  // 40960 or 20480
  static constexpr int A_COPIES = A_BYTES / 1024;      // 1-KB A copies per chunk (all waves)
  static constexpr int SB = MT == 128 ? 2 : 3;         // weight stages
  static constexpr int SMEM = 2 * A_BYTES + SB * PW_B_STAGE;
  static constexpr int EPI_BYTES = 16 * (8 * NCB + 4) * 4;  // per-wave gate/up epilogue staging
  static_assert(WM * 32 == MT && NCB % 4 == 0, "wave grid");
  static_assert(A_BYTES % 1024 == 0, "whole A copies");
  static_assert(PW_NW * EPI_BYTES <= SMEM, "epilogue staging fits the operand buffers");
  static_assert(SMEM + PW_NT * 4 <= 160 * 1024, "LDS");
};

// PACKED: the weights in the packed layout of moe_pack_weights (two weight
// rows' 64-byte chunk segments share one 128-byte line; each chunk's scale
// bytes are 4 per row, rows consecutive), so that a chunk's copies touch
// half the cache lines of the row-major codes and 1/32 of the lines of the
// row-major scales.  Same LDS contents, same arithmetic, same results.
template <bool GATEUP, int TERMS, bool PACKED, int MT>
__global__ __launch_bounds__(PW_NW * 64, 1) void expert_gemm_prefill_wide(GemmParams p, int spans) {
  // (the body is compiled for the device only: the host pass, which only
  // needs the kernel's signature for its launch stub, cannot type the
  // 6-register operands of the asm blocks)
#if defined(__HIP_DEVICE_COMPILE__)
  using C = PwCfg<MT>;
  constexpr int MB = 2, NCB = C::NCB, WN = C::WN;
  __shared__ __align__(16) uint8_t smem[C::SMEM];
  __shared__ float s_bias[PW_NT];

  // ---- work item: dealt to the XCDs in contiguous ranges ----
  const int total = *p.n_tiles * spans;
  const int per = (total + PF_XCD - 1) / PF_XCD;
  const int lin = blockIdx.x;
  const int item = (lin % PF_XCD) * per + lin / PF_XCD;
  if (lin / PF_XCD >= per || item >= total) return;
  const int tile = item / spans, span = item - tile * spans;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int rows = min(MT, p.counts[e] - m0);
  const int row_base = p.offsets[e] + m0;
  const int K = p.K, N = p.N, I = p.I, nblk = K >> 5;
  const int g = lane >> 4, r = lane & 15;

  // tile columns: gate/up -- gate columns span*256 .. +255 (tile rows
  // 0..255) and the same up columns (tile rows 256..511); down --
  // span*512 .. +511
  const int tcol0 = GATEUP ? span * (PW_NT / 2) : span * PW_NT;
  // tile row of the wave's column block j
  auto tile_row = [&](int j) -> int {
    if (GATEUP) return (j < NCB / 2 ? 0 : PW_NT / 2) + wn * (8 * NCB) + 16 * (j % (NCB / 2));
    return wn * (16 * NCB) + 16 * j;
  };
  // weight row (within the expert) of tile row n; rows past the output
  // take a row of the span's first block (never stored)
  auto weight_row = [&](int n) -> int {
    if (GATEUP) {
      const int c = tcol0 + (n % (PW_NT / 2));
      return gu_row(c < I ? c : tcol0 + (n & 15), n >= PW_NT / 2, I, p.alt);
    }
    const int c = tcol0 + n;
    return c < N ? c : tcol0 + (n & 15);
  };
  for (int n = tid; n < PW_NT; n += PW_NW * 64) {
    if (GATEUP) {
      const int c = min(tcol0 + (n % (PW_NT / 2)), I - 1);
      s_bias[n] = p.bias[(size_t)e * N + gu_row(c, n >= PW_NT / 2, I, p.alt)];
    } else {
      s_bias[n] = p.bias[(size_t)e * N + min(tcol0 + n, N - 1)];
    }
  }

  // ---- copy offsets (the chunk is added per chunk) ----
  const uint32_t a_rowbytes = (uint32_t)mx6_row_bytes(nblk);
  const uint32_t a_rows_total = GATEUP ? (uint32_t)p.T : (uint32_t)(p.T * p.k);
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.a, 0, (int)(a_rows_total * a_rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t crsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.b_codes, 0, (int)((uint32_t)p.E * (uint32_t)N * (uint32_t)(K >> 1)), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)p.b_scales, 0,
      (int)((uint32_t)p.E * (uint32_t)N * (uint32_t)(PACKED ? 4 * ((nblk + 3) >> 2) : nblk)), 0x00020000);
  constexpr uint32_t A_OOB = 0x7ffffff0u;  // at or past the A resource's end (it is below 2^31 bytes)
  // The copies are issued by the last CW waves only.  Issuing a chunk's
  // copies takes a wave several hundred cycles (the CU's address unit
  // accepts about 64 bytes a cycle), during which it issues no MFMAs; with
  // the copies on half the waves, the other wave of each SIMD keeps the
  // MFMA pipe busy meanwhile.  The copy waves are waves 4..7: the row
  // blocks that lie past the rows of a partly filled tile (2 and 3 of four
  // with 128-row tiles, 1 of two with 64-row tiles), so those waves have
  // nothing else to do there.
  constexpr int CW = PW_NW / 2;                          // copy waves
  constexpr int A_PW = (C::A_COPIES + CW - 1) / CW;      // A copies per copy wave
  constexpr int B_PW = PW_B_COPIES * PW_NW / CW;         // code copies per copy wave
  constexpr int S_PW = PW_S_COPIES * PW_NW / CW;         // row-major scale copies per copy wave
  constexpr int SP_PW = PW_NW / CW;                      // packed scale copies per copy wave
  const bool copier = wave >= PW_NW - CW;
  const int cw = copier ? wave - (PW_NW - CW) : 0;
  // A copy k of a copy wave (copy number i = CW k + cw of the chunk, if
  // below A_COPIES) fills LDS slots u = 64 i + lane: tile row u / 20, slot
  // u % 20 holding piece (u % 20) ^ ((row >> 1) & 3) (pieces of blocks past
  // K are copied from past the resource: zeros, so that those K positions
  // contribute nothing whatever the weights hold)
  uint32_t a_src[A_PW];
  int a_blk[A_PW];  // block of the piece within its group of four
#pragma unroll
  for (int k = 0; k < A_PW; ++k) {
    const int u = (CW * k + cw) * 64 + lane;
    const int m = u / 20, slot = u - 20 * m;
    const int piece = slot ^ ((m >> 1) & 3);
    uint32_t off = A_OOB;
    if (copier && m < rows) {
      const uint32_t arow = GATEUP ? (uint32_t)(p.expert_rows[(size_t)e * p.T + m0 + m] / p.k)
                                   : (uint32_t)(row_base + m);
      off = arow * a_rowbytes + (uint32_t)piece * 16u;
    }
    // (one term copies pieces 0, 1 and 4 only: the first term's codes and
    // the scale bytes; two terms pieces 0, 1, 2 and 4)
    a_src[k] = ((piece >> 2) > TERMS && (piece >> 2) < 4) ? A_OOB : off;
    a_blk[k] = piece & 3;
  }
  // B copy k of a copy wave fills slots u = (B_PW cw + k) * 64 + lane:
  // tile row u / 4, slot u % 4 holding block (u % 4) ^ ((n >> 2) & 3) of
  // the chunk
  uint32_t b_row[B_PW], b_odd[B_PW];
  int b_blk[B_PW];
#pragma unroll
  for (int k = 0; k < B_PW; ++k) {
    const int u = (B_PW * cw + k) * 64 + lane;
    const int n = u >> 2, slot = u & 3;
    const uint32_t wr = (uint32_t)weight_row(n);
    // row-major: the row's start; packed: its pair's start, plus 64 bytes
    // (one chunk segment) for the second row of the pair, scaled per chunk
    b_row[k] = PACKED ? ((uint32_t)e * (uint32_t)(N >> 1) + (wr >> 1)) * (uint32_t)K
                      : ((uint32_t)e * (uint32_t)N + wr) * (uint32_t)(K >> 1);
    b_odd[k] = wr & 1u;
    b_blk[k] = slot ^ ((n >> 2) & 3);
  }
  // A copy wave whose 16 B_PW tile rows all lie past the output (in the
  // last column span) issues no code copies with two weight stages, whose
  // wait drains every copy (vmcnt 0); those LDS rows keep stale codes, which
  // only the MFMA columns of discarded outputs read.  With three stages the
  // waits count every wave's copies, so all are issued.
  const int bn0 = 16 * B_PW * cw;
  const bool b_live = C::SB == 3 || (GATEUP ? tcol0 + (bn0 % (PW_NT / 2)) < I : tcol0 + bn0 < N);
  // row-major scale copy k of a copy wave fills dwords u = (S_PW cw + k)
  // * 64 + lane: tile row u / 2, block pair u % 2 of the chunk (two bytes,
  // low half of the dword)
  uint32_t s_row[PACKED ? 1 : S_PW];
  int s_pair[PACKED ? 1 : S_PW];
#pragma unroll
  for (int k = 0; k < (PACKED ? 0 : S_PW); ++k) {
    const int u = (S_PW * cw + k) * 64 + lane;
    s_row[k] = ((uint32_t)e * (uint32_t)N + (uint32_t)weight_row(u >> 1)) * (uint32_t)nblk;
    s_pair[k] = u & 1;
  }
  // packed scales: tile row n's four scale bytes of a chunk go to dword n
  // of the chunk's scale region.  Where the 512 tile rows are two runs of
  // 256 consecutive weight rows (the gate/up weight's gate-then-up layout,
  // and the down weight), copy waves 0 and 1 each move one run with a
  // single 16-byte copy (lane L: tile rows 256 cw + 4L .. +3; rows past the
  // output read on into other rows' scales, which only discarded outputs
  // use); with the interleaved gate/up layout every copy wave moves its
  // SP_PW groups of 64 rows with 4-byte copies (lane L of copy k: tile row
  // 64 j + L, j = SP_PW cw + k).
  const int nchk = (nblk + 3) >> 2;
  const bool sc16 = PACKED && !(GATEUP && p.alt);
  uint32_t sp_row[SP_PW];
#pragma unroll
  for (int k = 0; k < SP_PW; ++k) {
    const uint32_t run = GATEUP ? (uint32_t)(cw == 1 ? I : 0) + (uint32_t)tcol0 : (uint32_t)(tcol0 + 256 * cw);
    sp_row[k] = sc16 ? ((uint32_t)e * (uint32_t)nchk * (uint32_t)N + run) * 4u + 16u * (uint32_t)lane
                     : ((uint32_t)e * (uint32_t)nchk * (uint32_t)N + (uint32_t)weight_row(64 * (SP_PW * cw + k) + lane)) * 4u;
  }
  // A copies whose 3.2 tile rows all lie past the tile's rows (or past the
  // tile) are not issued: those LDS rows keep stale data, which only the
  // MFMA rows of discarded outputs read (an output row depends on its own A
  // row only)
  bool a_live[A_PW];
#pragma unroll
  for (int k = 0; k < A_PW; ++k)
    a_live[k] = CW * k + cw < C::A_COPIES && (CW * k + cw) * 64 / 20 < rows;
  auto issue_a = [&](int c, int stage) {
    if (!copier) return;
    uint8_t* base = smem + stage * C::A_BYTES;
#pragma unroll
    for (int k = 0; k < A_PW; ++k)
      if (a_live[k])
        lds_copy16(arsrc, (lds_void_t*)(base + (CW * k + cw) * 1024),
                   (a_src[k] == A_OOB || 4 * c + a_blk[k] >= nblk) ? A_OOB : a_src[k] + (uint32_t)c * MX6_GROUP_BYTES);
  };
  // the weight copies of a chunk: B_PW code copies, then the scale copies
  // (packed: one 16-byte copy on copy waves 0 and 1 and none on 2 and 3,
  // or SP_PW 4-byte copies; row-major: S_PW) per copy wave
  constexpr int B_OPS = B_PW + (PACKED ? SP_PW : S_PW);
  const int b_ops = sc16 ? B_PW + (cw < 2 ? 1 : 0) : B_OPS;  // (uniform)
  auto issue_b = [&](int c, int stage) {
    if (!copier) return;
    uint8_t* base = smem + 2 * C::A_BYTES + stage * PW_B_STAGE;
    if constexpr (PACKED) {
      // chunk c of a pair: 128 bytes (64 per row), or 2 x 16 (nblk - 4c)
      // bytes for a short last chunk; its blocks past K read on into the
      // next row or pair (finite codes, multiplied by zero A pieces)
      const uint32_t w = (uint32_t)(4 * c + 4 <= nblk ? 64 : 16 * (nblk - 4 * c));
      if (b_live) {
#pragma unroll
        for (int k = 0; k < B_PW; ++k)
          lds_copy16(crsrc, (lds_void_t*)(base + (B_PW * cw + k) * 1024),
                     b_row[k] + 128u * (uint32_t)c + b_odd[k] * w + (uint32_t)b_blk[k] * 16u);
      }
      if (sc16) {
        if (cw < 2)
          lds_copy16(srsrc, (lds_void_t*)(base + PW_B_BYTES + cw * 1024), sp_row[0] + (uint32_t)c * (uint32_t)N * 4u);
      } else {
#pragma unroll
        for (int k = 0; k < SP_PW; ++k)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, (lds_void_t*)(base + PW_B_BYTES + (SP_PW * cw + k) * 256),
                                                   4, sp_row[k] + (uint32_t)c * (uint32_t)N * 4u, 0, 0, 0);
      }
    } else {
      if (b_live) {
#pragma unroll
        for (int k = 0; k < B_PW; ++k)
          lds_copy16(crsrc, (lds_void_t*)(base + (B_PW * cw + k) * 1024),
                     b_row[k] + (uint32_t)min(4 * c + b_blk[k], nblk - 1) * 16u);
      }
#pragma unroll
      for (int k = 0; k < S_PW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            srsrc, (lds_void_t*)(base + PW_B_BYTES + (S_PW * cw + k) * 256), 2,
            s_row[k] + (uint32_t)min(4 * c + 2 * s_pair[k], nblk - 2), 0, 0, 0);
    }
  };

  v4f acc[MB][NCB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NCB; ++j) acc[mb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  // LDS byte offsets of this lane's fragments inside an A stage (a_lane)
  // and a weight stage (b_lane, s_lane): a lane part here, the row block /
  // piece / column block part as the instructions' offset fields.  A: row m = 32 wm + 16 mb + r, piece
  // 4q + g at slot (4q + g) ^ ((m >> 1) & 3) (the same for both row
  // blocks); B: row n = tile_row(j) + r, whose swizzle (n >> 2) & 3 is
  // (r >> 2) & 3; scales: byte g & 1 of dword 2n + g / 2.
  constexpr int WNR = GATEUP ? 8 * NCB : 16 * NCB;  // tile rows per column half
  const uint32_t a_lane = (uint32_t)((32 * wm + r) * MX6_GROUP_BYTES + 16 * (g ^ ((r >> 1) & 3)));
  const uint32_t b_lane = (uint32_t)((wn * WNR + r) * 64 + 16 * (g ^ ((r >> 2) & 3)));
  // scale bytes per tile row in LDS: row-major copies leave two bytes in
  // each of two dwords (8 per row), packed copies four bytes
  constexpr int SR = PACKED ? 4 : 8;
  const uint32_t s_lane = (uint32_t)(PW_B_BYTES + SR * (wn * WNR + r) +
                                     (PACKED ? g : 4 * (g >> 1) + (g & 1)));
  // tile row of column block j without the column half's part
  auto jrow = [](auto jc) constexpr {
    constexpr int j = decltype(jc)::value;
    return GATEUP ? (j < NCB / 2 ? 0 : PW_NT / 2) + 16 * (j % (NCB / 2)) : 16 * j;
  };

  constexpr int SB = C::SB;
  const int nchunk = (nblk + 3) >> 2;
  issue_a(0, 0);
  issue_b(0, 0);
  if (SB == 3 && nchunk > 1) issue_b(1, 1);
  int wst = 0;  // weight stage of chunk c (c mod SB)
  for (int c = 0; c < nchunk; ++c) {
    const uint32_t abase = (uint32_t)(uintptr_t)(smem + (c & 1) * C::A_BYTES);
    const uint32_t bbase = (uint32_t)(uintptr_t)(smem + 2 * C::A_BYTES + wst * PW_B_STAGE);
    // a copy wave's copies of chunk c: with three weight stages the weight
    // copies of chunk c+1, issued after the A copies of chunk c, may stay
    // in flight (vector memory loads complete in issue order)
    if (SB == 3 && c + 1 < nchunk) {
      if (b_ops == B_OPS)
        wait_vmcnt<B_OPS>();
      else if (b_ops == B_PW + 1)
        wait_vmcnt<B_PW + 1>();
      else
        wait_vmcnt<B_PW>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();  // everyone's copies of chunk c; everyone done with chunk c - 1
    __builtin_amdgcn_sched_barrier(0);
    // into the stages chunk c - 1 used
    if (c + 1 < nchunk) issue_a(c + 1, (c + 1) & 1);
    if (c + SB - 1 < nchunk) issue_b(c + SB - 1, wst == 0 ? SB - 1 : wst - 1);
    wst = wst == SB - 1 ? 0 : wst + 1;
    __builtin_amdgcn_sched_barrier(0);
    // a wave whose 32 rows all lie past the tile's rows (the last tile of
    // an expert) only copies and keeps the barriers: its SIMD's other wave
    // then has the MFMA pipe and the LDS port to itself
    if (32 * wm >= rows) continue;
    // A fragments (pieces 0..4 of block g of the lane's row in each row
    // block, zeros past K; one term reads pieces 0, 1 and 4, two terms 0, 1,
    // 2 and 4) and
    // the first group's B fragments, then the FP6 terms of A as 6-register
    // operands
    const uint32_t ab = abase + a_lane, bb = bbase + b_lane, sb = bbase + s_lane;
    v4u w[MB][5];
    v4u bq[2][4];
    uint32_t sq[2][4];
    if constexpr (TERMS == 3) {
      asm volatile(
        "ds_read_b128 %0, %18 offset:%21\n\t"
        "ds_read_b128 %1, %18 offset:%22\n\t"
        "ds_read_b128 %2, %18 offset:%23\n\t"
        "ds_read_b128 %3, %18 offset:%24\n\t"
        "ds_read_b128 %4, %18 offset:%25\n\t"
        "ds_read_b128 %5, %18 offset:%26\n\t"
        "ds_read_b128 %6, %18 offset:%27\n\t"
        "ds_read_b128 %7, %18 offset:%28\n\t"
        "ds_read_b128 %8, %18 offset:%29\n\t"
        "ds_read_b128 %9, %18 offset:%30\n\t"
        "ds_read_b128 %10, %19 offset:%31\n\t"
        "ds_read_b128 %11, %19 offset:%32\n\t"
        "ds_read_b128 %12, %19 offset:%33\n\t"
        "ds_read_b128 %13, %19 offset:%34\n\t"
        "ds_read_u8 %14, %20 offset:%35\n\t"
        "ds_read_u8 %15, %20 offset:%36\n\t"
        "ds_read_u8 %16, %20 offset:%37\n\t"
        "ds_read_u8 %17, %20 offset:%38\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0][0]), "=&v"(w[0][1]), "=&v"(w[0][2]), "=&v"(w[0][3]),
          "=&v"(w[0][4]), "=&v"(w[1][0]), "=&v"(w[1][1]), "=&v"(w[1][2]),
          "=&v"(w[1][3]), "=&v"(w[1][4]), "=&v"(bq[0][0]), "=&v"(bq[0][1]),
          "=&v"(bq[0][2]), "=&v"(bq[0][3]), "=&v"(sq[0][0]), "=&v"(sq[0][1]),
          "=&v"(sq[0][2]), "=&v"(sq[0][3])
        : "v"(ab), "v"(bb), "v"(sb),
          "i"(16 * MX6_GROUP_BYTES * 0 + 0), "i"(16 * MX6_GROUP_BYTES * 0 + 64), "i"(16 * MX6_GROUP_BYTES * 0 + 128),
          "i"(16 * MX6_GROUP_BYTES * 0 + 192), "i"(16 * MX6_GROUP_BYTES * 0 + 256), "i"(16 * MX6_GROUP_BYTES * 1 + 0),
          "i"(16 * MX6_GROUP_BYTES * 1 + 64), "i"(16 * MX6_GROUP_BYTES * 1 + 128), "i"(16 * MX6_GROUP_BYTES * 1 + 192),
          "i"(16 * MX6_GROUP_BYTES * 1 + 256), "i"(64 * jrow(std::integral_constant<int, 0>{})), "i"(64 * jrow(std::integral_constant<int, 1>{})),
          "i"(64 * jrow(std::integral_constant<int, 2>{})), "i"(64 * jrow(std::integral_constant<int, 3>{})), "i"(SR * jrow(std::integral_constant<int, 0>{})),
          "i"(SR * jrow(std::integral_constant<int, 1>{})), "i"(SR * jrow(std::integral_constant<int, 2>{})), "i"(SR * jrow(std::integral_constant<int, 3>{})));
    } else if constexpr (TERMS == 2) {
      asm volatile(
        "ds_read_b128 %0, %16 offset:%19\n\t"
        "ds_read_b128 %1, %16 offset:%20\n\t"
        "ds_read_b128 %2, %16 offset:%21\n\t"
        "ds_read_b128 %3, %16 offset:%22\n\t"
        "ds_read_b128 %4, %16 offset:%23\n\t"
        "ds_read_b128 %5, %16 offset:%24\n\t"
        "ds_read_b128 %6, %16 offset:%25\n\t"
        "ds_read_b128 %7, %16 offset:%26\n\t"
        "ds_read_b128 %8, %17 offset:%27\n\t"
        "ds_read_b128 %9, %17 offset:%28\n\t"
        "ds_read_b128 %10, %17 offset:%29\n\t"
        "ds_read_b128 %11, %17 offset:%30\n\t"
        "ds_read_u8 %12, %18 offset:%31\n\t"
        "ds_read_u8 %13, %18 offset:%32\n\t"
        "ds_read_u8 %14, %18 offset:%33\n\t"
        "ds_read_u8 %15, %18 offset:%34\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0][0]), "=&v"(w[0][1]), "=&v"(w[0][2]), "=&v"(w[0][4]), "=&v"(w[1][0]), "=&v"(w[1][1]),
          "=&v"(w[1][2]), "=&v"(w[1][4]), "=&v"(bq[0][0]), "=&v"(bq[0][1]), "=&v"(bq[0][2]), "=&v"(bq[0][3]),
          "=&v"(sq[0][0]), "=&v"(sq[0][1]), "=&v"(sq[0][2]), "=&v"(sq[0][3])
        : "v"(ab), "v"(bb), "v"(sb),
          "i"(16 * MX6_GROUP_BYTES * 0 + 0), "i"(16 * MX6_GROUP_BYTES * 0 + 64),
          "i"(16 * MX6_GROUP_BYTES * 0 + 128), "i"(16 * MX6_GROUP_BYTES * 0 + 256),
          "i"(16 * MX6_GROUP_BYTES * 1 + 0), "i"(16 * MX6_GROUP_BYTES * 1 + 64),
          "i"(16 * MX6_GROUP_BYTES * 1 + 128), "i"(16 * MX6_GROUP_BYTES * 1 + 256),
          "i"(64 * jrow(std::integral_constant<int, 0>{})), "i"(64 * jrow(std::integral_constant<int, 1>{})),
          "i"(64 * jrow(std::integral_constant<int, 2>{})), "i"(64 * jrow(std::integral_constant<int, 3>{})),
          "i"(SR * jrow(std::integral_constant<int, 0>{})), "i"(SR * jrow(std::integral_constant<int, 1>{})),
          "i"(SR * jrow(std::integral_constant<int, 2>{})), "i"(SR * jrow(std::integral_constant<int, 3>{})));
      w[0][3] = w[1][3] = (v4u){0u, 0u, 0u, 0u};
    } else {
      asm volatile(
        "ds_read_b128 %0, %14 offset:%17\n\t"
        "ds_read_b128 %1, %14 offset:%18\n\t"
        "ds_read_b128 %2, %14 offset:%19\n\t"
        "ds_read_b128 %3, %14 offset:%20\n\t"
        "ds_read_b128 %4, %14 offset:%21\n\t"
        "ds_read_b128 %5, %14 offset:%22\n\t"
        "ds_read_b128 %6, %15 offset:%23\n\t"
        "ds_read_b128 %7, %15 offset:%24\n\t"
        "ds_read_b128 %8, %15 offset:%25\n\t"
        "ds_read_b128 %9, %15 offset:%26\n\t"
        "ds_read_u8 %10, %16 offset:%27\n\t"
        "ds_read_u8 %11, %16 offset:%28\n\t"
        "ds_read_u8 %12, %16 offset:%29\n\t"
        "ds_read_u8 %13, %16 offset:%30\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0][0]), "=&v"(w[0][1]), "=&v"(w[0][4]), "=&v"(w[1][0]),
          "=&v"(w[1][1]), "=&v"(w[1][4]), "=&v"(bq[0][0]), "=&v"(bq[0][1]),
          "=&v"(bq[0][2]), "=&v"(bq[0][3]), "=&v"(sq[0][0]), "=&v"(sq[0][1]),
          "=&v"(sq[0][2]), "=&v"(sq[0][3])
        : "v"(ab), "v"(bb), "v"(sb),
          "i"(16 * MX6_GROUP_BYTES * 0 + 0), "i"(16 * MX6_GROUP_BYTES * 0 + 64), "i"(16 * MX6_GROUP_BYTES * 0 + 256),
          "i"(16 * MX6_GROUP_BYTES * 1 + 0), "i"(16 * MX6_GROUP_BYTES * 1 + 64), "i"(16 * MX6_GROUP_BYTES * 1 + 256),
          "i"(64 * jrow(std::integral_constant<int, 0>{})), "i"(64 * jrow(std::integral_constant<int, 1>{})), "i"(64 * jrow(std::integral_constant<int, 2>{})),
          "i"(64 * jrow(std::integral_constant<int, 3>{})), "i"(SR * jrow(std::integral_constant<int, 0>{})), "i"(SR * jrow(std::integral_constant<int, 1>{})),
          "i"(SR * jrow(std::integral_constant<int, 2>{})), "i"(SR * jrow(std::integral_constant<int, 3>{})));
      w[0][2] = w[0][3] = w[1][2] = w[1][3] = (v4u){0u, 0u, 0u, 0u};
    }
    v6u a6[MB][TERMS];
    uint32_t as[MB][TERMS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint32_t* x = (const uint32_t*)&w[mb][0];
#pragma unroll
      for (int t = 0; t < TERMS; ++t) {
        a6[mb][t] = (v6u){x[6 * t], x[6 * t + 1], x[6 * t + 2], x[6 * t + 3], x[6 * t + 4], x[6 * t + 5]};
        as[mb][t] = (x[18] >> (8 * t)) & 0xffu;
      }
    }
    // column-block groups of four: each asm block reads the next group's B
    // fragments while it issues this group's 8 * TERMS MFMAs (term-major, so
    // an accumulator's updates are eight MFMAs apart), then waits for the
    // reads.  s_nop: wait states for operands written just before by VALU
    // instructions.  Raised priority while the MFMAs issue, so that the other
    // wave of the SIMD (reading LDS meanwhile) does not interleave.
    StaticFor<0, NCB / 4>::run([&](auto gc) {
      constexpr int jg = decltype(gc)::value;
      constexpr int cur = jg & 1, nxt = cur ^ 1;
      if constexpr (TERMS == 3) {
        if constexpr (jg + 1 < NCB / 4) {
          constexpr int k0 = 4 * (jg + 1);
          asm volatile(
            "s_nop 4\n\t"
          "ds_read_b128 %8, %36 offset:%38\n\t"
          "ds_read_b128 %9, %36 offset:%39\n\t"
          "ds_read_b128 %10, %36 offset:%40\n\t"
          "ds_read_b128 %11, %36 offset:%41\n\t"
          "ds_read_u8 %12, %37 offset:%42\n\t"
          "ds_read_u8 %13, %37 offset:%43\n\t"
          "ds_read_u8 %14, %37 offset:%44\n\t"
          "ds_read_u8 %15, %37 offset:%45\n\t"
          "s_setprio 1\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %16, %28, %0, %22, %32 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %19, %28, %1, %25, %32 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %16, %29, %2, %22, %33 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %19, %29, %3, %25, %33 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %16, %30, %4, %22, %34 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %19, %30, %5, %25, %34 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %16, %31, %6, %22, %35 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %19, %31, %7, %25, %35 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %17, %28, %0, %23, %32 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %20, %28, %1, %26, %32 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %17, %29, %2, %23, %33 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %20, %29, %3, %26, %33 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %17, %30, %4, %23, %34 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %20, %30, %5, %26, %34 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %17, %31, %6, %23, %35 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %20, %31, %7, %26, %35 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %18, %28, %0, %24, %32 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %21, %28, %1, %27, %32 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %18, %29, %2, %24, %33 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %21, %29, %3, %27, %33 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %18, %30, %4, %24, %34 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %21, %30, %5, %27, %34 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %18, %31, %6, %24, %35 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %21, %31, %7, %27, %35 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "s_setprio 0\n\t"
          "s_waitcnt lgkmcnt(0)"
            : "+v"(acc[0][4 * jg]), "+v"(acc[1][4 * jg]), "+v"(acc[0][4 * jg + 1]), "+v"(acc[1][4 * jg + 1]),
            "+v"(acc[0][4 * jg + 2]), "+v"(acc[1][4 * jg + 2]), "+v"(acc[0][4 * jg + 3]), "+v"(acc[1][4 * jg + 3]),
              "=&v"(bq[nxt][0]), "=&v"(bq[nxt][1]), "=&v"(bq[nxt][2]), "=&v"(bq[nxt][3]),
              "=&v"(sq[nxt][0]), "=&v"(sq[nxt][1]), "=&v"(sq[nxt][2]), "=&v"(sq[nxt][3])
            : "v"(a6[0][0]), "v"(a6[0][1]), "v"(a6[0][2]), "v"(a6[1][0]), "v"(a6[1][1]), "v"(a6[1][2]),
              "v"(as[0][0]), "v"(as[0][1]), "v"(as[0][2]), "v"(as[1][0]), "v"(as[1][1]), "v"(as[1][2]),
              "v"(bq[cur][0]), "v"(bq[cur][1]), "v"(bq[cur][2]), "v"(bq[cur][3]),
              "v"(sq[cur][0]), "v"(sq[cur][1]), "v"(sq[cur][2]), "v"(sq[cur][3]), "v"(bb), "v"(sb),
              "i"(64 * jrow(std::integral_constant<int, k0>{})), "i"(64 * jrow(std::integral_constant<int, k0 + 1>{})),
              "i"(64 * jrow(std::integral_constant<int, k0 + 2>{})), "i"(64 * jrow(std::integral_constant<int, k0 + 3>{})),
              "i"(SR * jrow(std::integral_constant<int, k0>{})), "i"(SR * jrow(std::integral_constant<int, k0 + 1>{})),
              "i"(SR * jrow(std::integral_constant<int, k0 + 2>{})), "i"(SR * jrow(std::integral_constant<int, k0 + 3>{})));
        } else {
          asm volatile(
            "s_nop 4\n\t"
          "s_setprio 1\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %8, %20, %0, %14, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %11, %20, %1, %17, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %8, %21, %2, %14, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %11, %21, %3, %17, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %8, %22, %4, %14, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %11, %22, %5, %17, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %8, %23, %6, %14, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %11, %23, %7, %17, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %9, %20, %0, %15, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %12, %20, %1, %18, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %9, %21, %2, %15, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %12, %21, %3, %18, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %9, %22, %4, %15, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %12, %22, %5, %18, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %9, %23, %6, %15, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %12, %23, %7, %18, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %10, %20, %0, %16, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %13, %20, %1, %19, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %10, %21, %2, %16, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %13, %21, %3, %19, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %10, %22, %4, %16, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %13, %22, %5, %19, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %10, %23, %6, %16, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %13, %23, %7, %19, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "s_setprio 0"
            : "+v"(acc[0][4 * jg]), "+v"(acc[1][4 * jg]), "+v"(acc[0][4 * jg + 1]), "+v"(acc[1][4 * jg + 1]),
            "+v"(acc[0][4 * jg + 2]), "+v"(acc[1][4 * jg + 2]), "+v"(acc[0][4 * jg + 3]), "+v"(acc[1][4 * jg + 3])
            : "v"(a6[0][0]), "v"(a6[0][1]), "v"(a6[0][2]), "v"(a6[1][0]), "v"(a6[1][1]), "v"(a6[1][2]),
              "v"(as[0][0]), "v"(as[0][1]), "v"(as[0][2]), "v"(as[1][0]), "v"(as[1][1]), "v"(as[1][2]),
              "v"(bq[cur][0]), "v"(bq[cur][1]), "v"(bq[cur][2]), "v"(bq[cur][3]),
              "v"(sq[cur][0]), "v"(sq[cur][1]), "v"(sq[cur][2]), "v"(sq[cur][3]));
        }
      } else if constexpr (TERMS == 2) {
        if constexpr (jg + 1 < NCB / 4) {
          constexpr int k0 = 4 * (jg + 1);
          asm volatile(
            "s_nop 4\n\t"
          "ds_read_b128 %8, %32 offset:%34\n\t"
          "ds_read_b128 %9, %32 offset:%35\n\t"
          "ds_read_b128 %10, %32 offset:%36\n\t"
          "ds_read_b128 %11, %32 offset:%37\n\t"
          "ds_read_u8 %12, %33 offset:%38\n\t"
          "ds_read_u8 %13, %33 offset:%39\n\t"
          "ds_read_u8 %14, %33 offset:%40\n\t"
          "ds_read_u8 %15, %33 offset:%41\n\t"
          "s_setprio 1\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %16, %24, %0, %20, %28 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %18, %24, %1, %22, %28 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %16, %25, %2, %20, %29 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %18, %25, %3, %22, %29 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %16, %26, %4, %20, %30 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %18, %26, %5, %22, %30 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %16, %27, %6, %20, %31 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %18, %27, %7, %22, %31 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %17, %24, %0, %21, %28 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %19, %24, %1, %23, %28 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %17, %25, %2, %21, %29 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %19, %25, %3, %23, %29 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %17, %26, %4, %21, %30 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %19, %26, %5, %23, %30 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %17, %27, %6, %21, %31 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %19, %27, %7, %23, %31 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "s_setprio 0\n\t"
          "s_waitcnt lgkmcnt(0)"
            : "+v"(acc[0][4 * jg]), "+v"(acc[1][4 * jg]), "+v"(acc[0][4 * jg + 1]), "+v"(acc[1][4 * jg + 1]),
            "+v"(acc[0][4 * jg + 2]), "+v"(acc[1][4 * jg + 2]), "+v"(acc[0][4 * jg + 3]), "+v"(acc[1][4 * jg + 3]),
              "=&v"(bq[nxt][0]), "=&v"(bq[nxt][1]), "=&v"(bq[nxt][2]), "=&v"(bq[nxt][3]),
              "=&v"(sq[nxt][0]), "=&v"(sq[nxt][1]), "=&v"(sq[nxt][2]), "=&v"(sq[nxt][3])
            : "v"(a6[0][0]), "v"(a6[0][1]), "v"(a6[1][0]), "v"(a6[1][1]),
              "v"(as[0][0]), "v"(as[0][1]), "v"(as[1][0]), "v"(as[1][1]),
              "v"(bq[cur][0]), "v"(bq[cur][1]), "v"(bq[cur][2]), "v"(bq[cur][3]),
              "v"(sq[cur][0]), "v"(sq[cur][1]), "v"(sq[cur][2]), "v"(sq[cur][3]), "v"(bb), "v"(sb),
              "i"(64 * jrow(std::integral_constant<int, k0>{})), "i"(64 * jrow(std::integral_constant<int, k0 + 1>{})),
              "i"(64 * jrow(std::integral_constant<int, k0 + 2>{})), "i"(64 * jrow(std::integral_constant<int, k0 + 3>{})),
              "i"(SR * jrow(std::integral_constant<int, k0>{})), "i"(SR * jrow(std::integral_constant<int, k0 + 1>{})),
              "i"(SR * jrow(std::integral_constant<int, k0 + 2>{})), "i"(SR * jrow(std::integral_constant<int, k0 + 3>{})));
        } else {
          asm volatile(
            "s_nop 4\n\t"
          "s_setprio 1\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %8, %16, %0, %12, %20 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %10, %16, %1, %14, %20 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %8, %17, %2, %12, %21 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %10, %17, %3, %14, %21 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %8, %18, %4, %12, %22 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %10, %18, %5, %14, %22 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %8, %19, %6, %12, %23 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %10, %19, %7, %14, %23 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %9, %16, %0, %13, %20 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %11, %16, %1, %15, %20 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %9, %17, %2, %13, %21 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %11, %17, %3, %15, %21 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %9, %18, %4, %13, %22 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %11, %18, %5, %15, %22 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %9, %19, %6, %13, %23 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %11, %19, %7, %15, %23 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "s_setprio 0"
            : "+v"(acc[0][4 * jg]), "+v"(acc[1][4 * jg]), "+v"(acc[0][4 * jg + 1]), "+v"(acc[1][4 * jg + 1]),
            "+v"(acc[0][4 * jg + 2]), "+v"(acc[1][4 * jg + 2]), "+v"(acc[0][4 * jg + 3]), "+v"(acc[1][4 * jg + 3])
            : "v"(a6[0][0]), "v"(a6[0][1]), "v"(a6[1][0]), "v"(a6[1][1]),
              "v"(as[0][0]), "v"(as[0][1]), "v"(as[1][0]), "v"(as[1][1]),
              "v"(bq[cur][0]), "v"(bq[cur][1]), "v"(bq[cur][2]), "v"(bq[cur][3]),
              "v"(sq[cur][0]), "v"(sq[cur][1]), "v"(sq[cur][2]), "v"(sq[cur][3]));
        }
      } else {
        if constexpr (jg + 1 < NCB / 4) {
          constexpr int k0 = 4 * (jg + 1);
          asm volatile(
            "s_nop 4\n\t"
          "ds_read_b128 %8, %28 offset:%30\n\t"
          "ds_read_b128 %9, %28 offset:%31\n\t"
          "ds_read_b128 %10, %28 offset:%32\n\t"
          "ds_read_b128 %11, %28 offset:%33\n\t"
          "ds_read_u8 %12, %29 offset:%34\n\t"
          "ds_read_u8 %13, %29 offset:%35\n\t"
          "ds_read_u8 %14, %29 offset:%36\n\t"
          "ds_read_u8 %15, %29 offset:%37\n\t"
          "s_setprio 1\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %16, %20, %0, %18, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %17, %20, %1, %19, %24 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %16, %21, %2, %18, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %17, %21, %3, %19, %25 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %16, %22, %4, %18, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %17, %22, %5, %19, %26 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %16, %23, %6, %18, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %17, %23, %7, %19, %27 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "s_setprio 0\n\t"
          "s_waitcnt lgkmcnt(0)"
            : "+v"(acc[0][4 * jg]), "+v"(acc[1][4 * jg]), "+v"(acc[0][4 * jg + 1]), "+v"(acc[1][4 * jg + 1]),
            "+v"(acc[0][4 * jg + 2]), "+v"(acc[1][4 * jg + 2]), "+v"(acc[0][4 * jg + 3]), "+v"(acc[1][4 * jg + 3]),
              "=&v"(bq[nxt][0]), "=&v"(bq[nxt][1]), "=&v"(bq[nxt][2]), "=&v"(bq[nxt][3]),
              "=&v"(sq[nxt][0]), "=&v"(sq[nxt][1]), "=&v"(sq[nxt][2]), "=&v"(sq[nxt][3])
            : "v"(a6[0][0]), "v"(a6[1][0]),
              "v"(as[0][0]), "v"(as[1][0]),
              "v"(bq[cur][0]), "v"(bq[cur][1]), "v"(bq[cur][2]), "v"(bq[cur][3]),
              "v"(sq[cur][0]), "v"(sq[cur][1]), "v"(sq[cur][2]), "v"(sq[cur][3]), "v"(bb), "v"(sb),
              "i"(64 * jrow(std::integral_constant<int, k0>{})), "i"(64 * jrow(std::integral_constant<int, k0 + 1>{})),
              "i"(64 * jrow(std::integral_constant<int, k0 + 2>{})), "i"(64 * jrow(std::integral_constant<int, k0 + 3>{})),
              "i"(SR * jrow(std::integral_constant<int, k0>{})), "i"(SR * jrow(std::integral_constant<int, k0 + 1>{})),
              "i"(SR * jrow(std::integral_constant<int, k0 + 2>{})), "i"(SR * jrow(std::integral_constant<int, k0 + 3>{})));
        } else {
          asm volatile(
            "s_nop 4\n\t"
          "s_setprio 1\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %8, %12, %0, %10, %16 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %1, %9, %12, %1, %11, %16 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %2, %8, %13, %2, %10, %17 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %3, %9, %13, %3, %11, %17 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %4, %8, %14, %4, %10, %18 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %5, %9, %14, %5, %11, %18 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %6, %8, %15, %6, %10, %19 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "v_mfma_scale_f32_16x16x128_f8f6f4 %7, %9, %15, %7, %11, %19 op_sel_hi:[0,0,0] cbsz:2 blgp:4\n\t"
          "s_setprio 0"
            : "+v"(acc[0][4 * jg]), "+v"(acc[1][4 * jg]), "+v"(acc[0][4 * jg + 1]), "+v"(acc[1][4 * jg + 1]),
            "+v"(acc[0][4 * jg + 2]), "+v"(acc[1][4 * jg + 2]), "+v"(acc[0][4 * jg + 3]), "+v"(acc[1][4 * jg + 3])
            : "v"(a6[0][0]), "v"(a6[1][0]),
              "v"(as[0][0]), "v"(as[1][0]),
              "v"(bq[cur][0]), "v"(bq[cur][1]), "v"(bq[cur][2]), "v"(bq[cur][3]),
              "v"(sq[cur][0]), "v"(sq[cur][1]), "v"(sq[cur][2]), "v"(sq[cur][3]));
        }
      }
    });
  }
  // wait states before anything reads the accumulators the MFMAs wrote
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __syncthreads();  // every wave is done with the operand buffers

  float bias[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) bias[j] = s_bias[tile_row(j) + r];
  const int rows_w = rows - 32 * wm;
  const int row_base_w = row_base + 32 * wm;
  const int wcol0 = GATEUP ? tcol0 + wn * (8 * NCB) : tcol0 + wn * (16 * NCB);
  uint8_t* scratch = smem + wave * C::EPI_BYTES;
  if (rows_w <= 0) return;
  if (GATEUP)
    pf_epilogue_gateup<NCB>(p, acc, bias, rows_w, row_base_w, wcol0, lane, scratch);
  else
    pf_epilogue_down<NCB>(p, acc, bias, rows_w, row_base_w, wcol0, lane, scratch);
#endif
}

static bool prefill_offsets_fit(const GemmParams& p) {
  const unsigned long long lim = 1ull << 32;
  const unsigned long long a_rows = p.hq ? (unsigned long long)p.T : (unsigned long long)p.T * p.k;
  const unsigned long long e_rows = (unsigned long long)p.E * p.N;
  return a_rows * mx6_row_bytes(p.K / 32) < lim && e_rows * (p.K / 2) < lim;
}

// A launch, optionally with start and stop events that the launch itself
// records when the kernel starts and ends (no dispatch time between them).
template <typename K, typename... A>
static void launch_k(K kernel, dim3 g, dim3 b, hipStream_t s, const LaunchEvents& ev, A... args) {
  if (ev.start && ev.stop)
    hipExtLaunchKernelGGL(kernel, g, b, 0, s, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, g, b, 0, s, args...);
}

// Decode kernel instance for the phase count of K (unrolled up to 8 phases).
template <bool GATEUP, bool U16, int TERMS, int MB, bool PACKED>
static void launch_decode_u(const GemmParams& p, unsigned grid, int spans, hipStream_t s, const LaunchEvents& ev) {
  const int nph = (p.K / 32 + DEC_KPH - 1) / DEC_KPH;
  const dim3 g(grid), b(DEC_NW * 64);
#define MOE_DEC(NPH) launch_k(expert_gemm_decode<GATEUP, NPH, U16, TERMS, MB, PACKED>, g, b, s, ev, p, spans)
  switch (nph) {
    case 1: MOE_DEC(1); break;
    case 2: MOE_DEC(2); break;
    case 3: MOE_DEC(3); break;
    case 4: MOE_DEC(4); break;
    case 5: MOE_DEC(5); break;
    case 6: MOE_DEC(6); break;
    case 7: MOE_DEC(7); break;
    case 8: MOE_DEC(8); break;
    default: MOE_DEC(0); break;
  }
#undef MOE_DEC
}

template <bool GATEUP, int TERMS, int MB>
static void launch_decode_mb(const GemmParams& p, unsigned items, int spans, hipStream_t s, const LaunchEvents& ev) {
  if (p.packed)  // (the packed layout has K/32 even)
    launch_decode_u<GATEUP, true, TERMS, MB, true>(p, items, spans, s, ev);
  else if ((p.K / 32) % 2 == 0)
    launch_decode_u<GATEUP, true, TERMS, MB, false>(p, items, spans, s, ev);
  else
    launch_decode_u<GATEUP, false, TERMS, MB, false>(p, items, spans, s, ev);
}

template <bool GATEUP, int TERMS>
static void launch_decode(const GemmParams& p, unsigned items, int spans, hipStream_t s, const LaunchEvents& ev) {
  if (p.mb == 2)
    launch_decode_mb<GATEUP, TERMS, 2>(p, items, spans, s, ev);
  else
    launch_decode_mb<GATEUP, TERMS, 1>(p, items, spans, s, ev);
}

template <bool GATEUP, int TERMS>
static int launch_gemm(const GemmParams& p, int max_tiles, int mode, hipStream_t s, const LaunchEvents& ev) {
  const int n_out = GATEUP ? p.I : p.N;  // output columns
  if (mode == GEMM_DECODE) {
    const int spans = GATEUP ? (n_out + 31) / 32 : (n_out + 63) / 64;
    launch_decode<GATEUP, TERMS>(p, (unsigned)((long long)max_tiles * spans), spans, s, ev);
  } else {
    if (!prefill_offsets_fit(p)) return -1;
    const bool wide = mode == GEMM_WIDE || mode == GEMM_WIDE64;
    const int span_cols = wide ? (GATEUP ? PW_NT / 2 : PW_NT) : (GATEUP ? PF_NT / 2 : PF_NT);
    const int spans = (n_out + span_cols - 1) / span_cols;
    const long long items = (long long)max_tiles * spans;
    const dim3 g((unsigned)((items + PF_XCD - 1) / PF_XCD * PF_XCD));
#define MOE_WIDE(PK, MT) launch_k(expert_gemm_prefill_wide<GATEUP, TERMS, PK, MT>, g, dim3(PW_NW * 64), s, ev, p, spans)
    if (mode == GEMM_WIDE64) {
      if (p.packed) MOE_WIDE(true, 64); else MOE_WIDE(false, 64);
    } else if (wide) {
      if (p.packed) MOE_WIDE(true, 128); else MOE_WIDE(false, 128);
    } else
      launch_k(expert_gemm_prefill<GATEUP, TERMS>, g, dim3(PF_NW * 64), s, ev, p, spans);
#undef MOE_WIDE
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Launch configurations.
//   small-M (tiles of 16 rows, decode): one workgroup per (tile, 64-row
//     span) item, four waves stream the span's weights through LDS;
//   large-M (prefill): one workgroup per (64-row tile, 256-column span)
//     work item, 1-D grid dealt to the XCDs in contiguous ranges;
//   wide (prefill with enough rows per expert and even K/32 for both
//     projections): one workgroup per (128-row tile, 512-column span);
//   wide64 (the same with 33 to 48 rows per expert on average): one
//     workgroup per (64-row tile, 512-column span), three weight stages.
// p.terms: 3 (the exact path), 2 (the two-term option) or 1 (the
// activation-quantised fast mode).
int launch_gemm_gateup(const GemmParams& p, int max_tiles, int mode, hipStream_t s, const LaunchEvents& ev) {
  if (p.terms == 1) return launch_gemm<true, 1>(p, max_tiles, mode, s, ev);
  if (p.terms == 2) return launch_gemm<true, 2>(p, max_tiles, mode, s, ev);
  if (p.terms == 3) return launch_gemm<true, 3>(p, max_tiles, mode, s, ev);
  return -1;
}

int launch_gemm_down(const GemmParams& p, int max_tiles, int mode, hipStream_t s, const LaunchEvents& ev) {
  if (p.terms == 1) return launch_gemm<false, 1>(p, max_tiles, mode, s, ev);
  if (p.terms == 2) return launch_gemm<false, 2>(p, max_tiles, mode, s, ev);
  if (p.terms == 3) return launch_gemm<false, 3>(p, max_tiles, mode, s, ev);
  return -1;
}

}  // namespace moe
