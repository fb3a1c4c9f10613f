// The attention steps beside the MoE layer ("OpenAI 最新开源模型 gpt-oss 架构与训练
// 解析", 模型架构: Attention item; same page, "RoPE 替换了绝对位置编码" and
// "Attention Bias and Attention Sinks"):
//
//   rope_kernel  rotary encoding of query or key rows: the pair
//                (x[2i], x[2i+1]) of every head turns by pos * 10000^(-2i/D);
//   attn_kernel  grouped-query attention (the G = Hq / Hkv consecutive query
//                heads of a group read one key/value head), causal, optionally
//                limited to the band of the last `window` positions, with each
//                head's sink logit as one more term of the softmax denominator.
//
// attn_kernel is a one-pass (online-softmax) attention on bf16 MFMAs
// (v_mfma_f32_16x16x32_bf16) for head width 64.  A wave owns NQ blocks of 16
// query columns; column c of a block is (position c / G, head c % G) of one
// key/value group, so the G heads that share a key tile share its MFMAs.  Per
// tile of 32 keys:
//   S^T = K Q^T      A = 16 keys x 32 head elements (16-byte LDS reads),
//                    B = the lane's query column (registers, loaded once);
//                    the C layout puts one query column in each lane and four
//                    keys of it in each of the four lane groups;
//   softmax          scores scaled by log2(e)/sqrt(D), masked, running max and
//                    sum per column (exchanged between the four lane groups);
//   O^T += V^T P^T   A = 16 head elements x 32 keys, read from the value tile
//                    (stored as it comes, key rows) with gfx950's transposing
//                    LDS reads, B = P^T straight from the softmax's registers
//                    (the MFMA's K order is chosen to match them).
//                    P is fed as two bf16 terms, hi = bf16(p) and
//                    lo = bf16(p - hi), so the products carry p to about 2^-17.
// The output O^T has the same one-column-per-lane layout as the softmax
// state, so rescaling needs no data movement.
//
// Two launch shapes:
//   query split (KS = false): four waves own 4 * NQ blocks of columns and
//     share every key/value tile, which the workgroup stages in LDS (double
//     buffered, one barrier per tile, three tiles' loads in flight);
//   key split (KS = true, a workgroup's positions fit one wave, as in decode):
//     eight waves own the same columns and take every eighth tile each,
//     each staging its own tiles (two tiles' loads in flight); their partial
//     states are merged at the end in wave order, so the result does not
//     depend on timing.
// Tiles that every column of a wave sees whole skip the masking.
#include "moe_common.h"
#include "moe_kernels.h"

#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "attention.hip is written for gfx950 only"
#endif

namespace moe {

constexpr int AT_D = 64;              // head width
constexpr int AT_BK = 32;             // keys per tile
constexpr int AT_NQ = 2;              // 16-column blocks per wave
constexpr int AT_TILE_BYTES = AT_BK * AT_D * 2;  // 4 KB of keys or of values

// LDS copy of one tile: keys and values as rows of 128 bytes (one key each),
// their 16-byte chunks XOR-swizzled -- keys by the key's bits 0..2, values by
// bits 1..3 -- so that the 16-byte key reads are conflict-free and the
// values' transposing 8-byte reads (16 rows at a time) at most two-way.
struct AttnTile {
  uint8_t k[AT_TILE_BYTES];
  uint8_t v[AT_TILE_BYTES];
};

__device__ __forceinline__ uint32_t k_lds_off(int key, int chunk) { return key * 128 + ((chunk ^ (key & 7)) << 4); }
// byte offset of the 8-byte group q (head elements 4q .. 4q+3) of key `key`
__device__ __forceinline__ uint32_t v_lds_off(int key, int q) {
  return key * 128 + ((((q >> 1) ^ ((key >> 1) & 7))) << 4) + ((q & 1) << 3);
}

typedef short at_s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) at_s4 lds_s4;

// gfx950's transposing LDS read (ds_read_b64_tr_b16): within each group of
// 16 lanes, if lane 4i + s reads the 4 elements D[4i + s][0..3] at its
// address, lane j receives D[4i + j / 4][j % 4] for i = 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* p) {
  const at_s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(__attribute__((address_space(3))) uint8_t*)p);
  return __builtin_bit_cast(uint2, v);
}

// Copies the 16-byte chunks u = first, first + step, ... (< 256) of tile t
// (keys 32t .. 32t + 31 of key/value head hk of sequence b) from registers
// into the LDS tile; chunk u is key u >> 3, head elements 8 (u & 7) .. + 7.
template <int NCH>
struct TileRegs {
  uint4 k[NCH], v[NCH];
};

template <int NCH>
__device__ __forceinline__ void tile_load(const AttnParams& p, int b, int hk, int t, int first, int step,
                                          TileRegs<NCH>& r) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int u = first + i * step, key = AT_BK * t + (u >> 3), c = u & 7;
    if (key < p.S) {
      const size_t off = (((size_t)b * p.S + key) * p.Hkv + hk) * AT_D + 8 * c;
      r.k[i] = *(const uint4*)(p.k + off);
      r.v[i] = *(const uint4*)(p.v + off);
    } else {
      r.k[i] = make_uint4(0u, 0u, 0u, 0u);
      r.v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

template <int NCH>
__device__ __forceinline__ void tile_store(AttnTile& s, int first, int step, const TileRegs<NCH>& r) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int u = first + i * step, key = u >> 3, c = u & 7;
    *(uint4*)(s.k + k_lds_off(key, c)) = r.k[i];
    *(uint4*)(s.v + v_lds_off(key, 2 * c)) = r.v[i];
  }
}

typedef float at_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 at_b2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((at_f2){a, b}, at_b2));
}

// Reductions over the four lanes r, r + 16, r + 32, r + 48 (one query column):
// gfx950's permlane swaps hand each lane the values of the lane pair
// {l, l ^ 16} (then {l, l ^ 32}) in their two results, in either order.
__device__ __forceinline__ float col_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Running softmax state of the lane's NQ query columns and their O^T blocks
// (head elements 16 db + 4 g .. + 3 of column r of block n in acc[n][db]).
struct AttnState {
  float m[AT_NQ], l[AT_NQ];
  v4f acc[AT_NQ][AT_D / 16];
};

// One tile for the lane's NQ column blocks.  pos[n] is the position of the
// lane's column in block n (-1 for columns past the batch, so that all their
// keys are masked); a column sees key j when 0 <= pos - j < span.  MASK =
// false for a tile every column of the wave sees whole (the caller checks
// that), which skips the masking.
template <bool MASK>
__device__ __forceinline__ void attn_tile(const AttnTile& s, int t, const v8bf (&qf)[AT_NQ][2],
                                          const int (&pos)[AT_NQ], const bool (&live)[AT_NQ], uint32_t span,
                                          float scale, AttnState& st) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  // K fragments: key 16 kb + r, head elements 32 ks + 8 g .. + 7
  v8bf kf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      kf[kb][ks] = *(const v8bf*)(s.k + k_lds_off(16 * kb + r, 4 * ks + g));
  // V^T fragments: head element 16 db + r, keys 4g .. 4g+3 and 16+4g ..
  // 16+4g+3.  Lane (g, 4i + s) reads elements 16 db + 4s .. + 3 of key
  // 4g + i (then of key 16 + 4g + i); the transposing read hands lane
  // (g, r) element 16 db + r of the four keys.
  v8bf vf[AT_D / 16];
  const int ki = r >> 2, qs = r & 3;
#pragma unroll
  for (int db = 0; db < AT_D / 16; ++db) {
    const uint2 a = lds_read_tr16(s.v + v_lds_off(4 * g + ki, 4 * db + qs));
    const uint2 c = lds_read_tr16(s.v + v_lds_off(16 + 4 * g + ki, 4 * db + qs));
    vf[db] = __builtin_bit_cast(v8bf, make_uint4(a.x, a.y, c.x, c.y));
  }
#pragma unroll
  for (int n = 0; n < AT_NQ; ++n) {
    // a block whose columns are all past the batch (decode) is skipped whole
    if (n > 0 && !__builtin_amdgcn_ballot_w64(live[n])) continue;
    v4f sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][ks], qf[n][ks], sc[kb], 0, 0, 0);
    }
    // mask; key of sc[kb][e] is 32 t + 16 kb + 4 g + e.  The running max is
    // kept in scaled (log2) units; the scale is positive, so the max of the
    // raw scores is taken first and scaled once.
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = AT_BK * t + 16 * kb + 4 * g + e;
        // (one unsigned compare: 0 <= pos - key < span, span the band's
        // width or 2^31 - 1; columns past the batch have pos = -1)
        const bool ok = !MASK || (uint32_t)(pos[n] - key) < span;
        const float v = ok ? sc[kb][e] : -INFINITY;
        x[4 * kb + e] = v;
        mx = fmaxf(mx, v);
      }
    mx = col_max(mx);
    // The reference point of the exponentials moves only when the column's
    // max passes it by more than 2^8: the weights then stay below 256 (well
    // inside fp32, and the two-term bf16 split is relative), and most tiles
    // leave the output unscaled.  (The hardware exp2: results below 2^-126
    // flush to zero, negligible next to the running sum.)
    const float mcand = fmaxf(st.m[n], mx * scale);
    const float mnew = mcand > st.m[n] + 8.f ? mcand : st.m[n];
    float alpha, ps = 0.f;
    uint32_t hi[4], lo[4];
    if (MASK && mnew == -INFINITY) {  // no key and no finite sink yet
      alpha = 1.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) hi[e] = lo[e] = 0u;
    } else {
      alpha = __builtin_amdgcn_exp2f(st.m[n] - mnew);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(x[e], scale, -mnew));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(x[e + 1], scale, -mnew));
        ps += p0 + p1;
        const uint32_t h = pack_bf16x2(p0, p1);
        hi[e >> 1] = h;
        lo[e >> 1] = pack_bf16x2(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
      }
    }
    ps = col_sum(ps);
    st.l[n] = st.l[n] * alpha + ps;
    st.m[n] = mnew;
    const v8bf phi = __builtin_bit_cast(v8bf, make_uint4(hi[0], hi[1], hi[2], hi[3]));
    const v8bf plo = __builtin_bit_cast(v8bf, make_uint4(lo[0], lo[1], lo[2], lo[3]));
    // rescale the output only when some column's reference point moved
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db) st.acc[n][db] *= alpha;
    }
#pragma unroll
    for (int db = 0; db < AT_D / 16; ++db) {
      const v4f a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], phi, st.acc[n][db], 0, 0, 0);
      st.acc[n][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], plo, a, 0, 0, 0);
    }
  }
}

// Waves per workgroup and tiles whose loads are in flight ahead of the one
// being computed, per launch shape.
template <bool KS>
struct AttnShape {
  static constexpr int NW = KS ? 8 : 4;
  static constexpr int PF = KS ? 2 : 3;
  static constexpr int NCH = KS ? 4 : 1;      // 16-byte chunks of keys (and of values) a thread loads per tile
};

template <int G, bool KS>
__global__ __launch_bounds__(AttnShape<KS>::NW * 64) void attn_kernel(AttnParams p) {
  constexpr int NW = AttnShape<KS>::NW, PF = AttnShape<KS>::PF, NCH = AttnShape<KS>::NCH;
  constexpr int PPB = 16 / G;            // positions per column block
  constexpr int PPW = AT_NQ * PPB;       // positions per wave
  constexpr int QB = KS ? PPW : NW * PPW;  // positions per workgroup
  // query split: two tiles (double buffer); key split: one per wave, whose
  // space then holds the wave's O^T for the merge (64 lanes x 32 floats)
  __shared__ AttnTile s_tile[KS ? NW : 2];
  __shared__ float s_ml[KS ? NW : 1][KS ? 64 : 1][2 * AT_NQ];
  static_assert(!KS || 64 * AT_NQ * AT_D / 4 * 4 <= (int)sizeof(AttnTile), "O^T fits the wave's tile");

  const int b = blockIdx.z, hk = blockIdx.y;
  // causal work grows with the position: the last blocks go first
  const int qb = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int i0 = qb * QB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;

  // the lane's query columns and their fragments (B operand of S^T)
  int pos[AT_NQ], qi[AT_NQ];
  bool live[AT_NQ];
  v8bf qf[AT_NQ][2];
  const int h = hk * G + r % G;
  const int wq0 = i0 + (KS ? 0 : wave * PPW);  // the wave's first query
#pragma unroll
  for (int n = 0; n < AT_NQ; ++n) {
    qi[n] = wq0 + n * PPB + r / G;
    live[n] = qi[n] < p.Tq;
    pos[n] = live[n] ? p.q_pos0 + qi[n] : -1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (live[n]) w = *(const uint4*)(p.q + (((size_t)b * p.Tq + qi[n]) * p.Hq + h) * AT_D + 32 * ks + 8 * g);
      qf[n][ks] = __builtin_bit_cast(v8bf, w);
    }
  }
  // tiles that every column of the wave sees whole need no mask
  const bool wave_full = wq0 + PPW <= p.Tq;
  const int wp0 = p.q_pos0 + wq0, wp1 = wp0 + PPW - 1;
  const uint32_t span = p.window > 0 ? (uint32_t)p.window : 0x7fffffffu;
  auto unmasked = [&](int t) {
    return wave_full && AT_BK * t + AT_BK - 1 <= wp0 && (p.window == 0 || wp1 - AT_BK * t < p.window);
  };
  auto tile = [&](const AttnTile& s, int t, AttnState& st) {
    if (unmasked(t))
      attn_tile<false>(s, t, qf, pos, live, span, p.qk_scale, st);
    else
      attn_tile<true>(s, t, qf, pos, live, span, p.qk_scale, st);
  };
  // the sink starts the running state of one wave per column (all in the
  // query split, wave 0 in the key split)
  const float sink = p.sinks[h] * 1.4426950408889634f;
  AttnState st;
#pragma unroll
  for (int n = 0; n < AT_NQ; ++n) {
    const bool own = !KS || wave == 0;
    st.m[n] = own ? sink : -INFINITY;
    st.l[n] = (own && sink > -INFINITY) ? 1.f : 0.f;
#pragma unroll
    for (int db = 0; db < AT_D / 16; ++db) st.acc[n][db] = (v4f){0.f, 0.f, 0.f, 0.f};
  }

  // keys any of the workgroup's positions can see
  const int pmin = p.q_pos0 + i0;
  const int pmax = p.q_pos0 + min(i0 + QB, p.Tq) - 1;
  const int lo = p.window > 0 ? max(0, pmin - p.window + 1) : 0;
  const int t0 = lo / AT_BK, t1 = pmax / AT_BK;

  // a ring of PF tiles in registers: the loads of tile t + PF are issued
  // once tile t has left its registers
  TileRegs<NCH> rg[PF];
  if constexpr (!KS) {
    // query split: all threads stage each tile (one chunk of keys and one of
    // values each) into one of two LDS buffers, one barrier per tile
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (t0 + j <= t1) tile_load<NCH>(p, b, hk, t0 + j, tid, NW * 64, rg[j]);
    for (int tb = t0; tb <= t1; tb += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int t = tb + j;
        if (t > t1) break;
        AttnTile& s = s_tile[(t - t0) & 1];
        tile_store<NCH>(s, tid, NW * 64, rg[j]);
        __syncthreads();  // tile t staged; every wave is done with tile t - 2's buffer
        if (t + PF <= t1) tile_load<NCH>(p, b, hk, t + PF, tid, NW * 64, rg[j]);
        tile(s, t, st);
      }
    }
  } else {
    // key split: wave w takes tiles t0 + w, t0 + w + NW, ..., staging each in
    // its own LDS tile (the 64 lanes load four chunks of keys and four of
    // values each)
    AttnTile& s = s_tile[wave];
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (t0 + wave + j * NW <= t1) tile_load<NCH>(p, b, hk, t0 + wave + j * NW, lane, 64, rg[j]);
    for (int tb = t0 + wave; tb <= t1; tb += PF * NW) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int t = tb + j * NW;
        if (t > t1) break;
        tile_store<NCH>(s, lane, 64, rg[j]);
        if (t + PF * NW <= t1) tile_load<NCH>(p, b, hk, t + PF * NW, lane, 64, rg[j]);
        tile(s, t, st);
      }
    }
    // merge the waves' states in wave order: m and l in s_ml, O^T in the
    // wave's own tile space
    float* acc_out = (float*)&s_tile[wave] + lane * (AT_NQ * AT_D / 4);
#pragma unroll
    for (int n = 0; n < AT_NQ; ++n) {
      s_ml[wave][lane][n] = st.m[n];
      s_ml[wave][lane][AT_NQ + n] = st.l[n];
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc_out[(n * (AT_D / 16) + db) * 4 + e] = st.acc[n][db][e];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int n = 0; n < AT_NQ; ++n) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, s_ml[w][lane][n]);
      float L = 0.f;
      v4f O[AT_D / 16];
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db) O[db] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_ml[w][lane][n];
        const float f = (M == -INFINITY || mw == -INFINITY) ? 0.f : exp2f(mw - M);
        L += s_ml[w][lane][AT_NQ + n] * f;
        const float* aw = (const float*)&s_tile[w] + lane * (AT_NQ * AT_D / 4);
#pragma unroll
        for (int db = 0; db < AT_D / 16; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) O[db][e] += aw[(n * (AT_D / 16) + db) * 4 + e] * f;
      }
      st.l[n] = L;
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db) st.acc[n][db] = O[db];
    }
  }

  // out[b][qi][h][16 db + 4 g + e] = bf16(O / l)
#pragma unroll
  for (int n = 0; n < AT_NQ; ++n) {
    if (!live[n]) continue;
    const float inv = 1.0f / st.l[n];
    uint16_t* o = p.out + (((size_t)b * p.Tq + qi[n]) * p.Hq + h) * AT_D + 4 * g;
#pragma unroll
    for (int db = 0; db < AT_D / 16; ++db) {
      const v4f a = st.acc[n][db];
      *(uint2*)(o + 16 * db) = make_uint2(pack_bf16x2(a[0] * inv, a[1] * inv), pack_bf16x2(a[2] * inv, a[3] * inv));
    }
  }
}

// Rotary encoding: one thread per (row, pair), all heads of the row.  The
// angle pos * theta^(-2i/D) is formed and reduced to [-pi, pi] in double
// precision, so long positions keep their accuracy; the rotation itself is
// fp32, rounded once to bf16.
__global__ __launch_bounds__(256) void rope_kernel(const uint16_t* x, uint16_t* out, int n, int H, int D, int pos0,
                                                   double log2_theta) {
  const int half = D >> 1;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)n * half) return;
  const int t = (int)(idx / half), i = (int)(idx - (long long)t * half);
  const double inv = exp2(-2.0 * (double)i / (double)D * log2_theta);
  const double ang = (double)(pos0 + t) * inv;
  const double two_pi = 6.283185307179586476925;
  const double red = ang - two_pi * rint(ang / two_pi);
  float sn, cs;
  sincosf((float)red, &sn, &cs);
  const uint32_t* xr = (const uint32_t*)x + (size_t)t * H * half + i;
  uint32_t* orow = (uint32_t*)out + (size_t)t * H * half + i;
  for (int hh = 0; hh < H; ++hh) {
    const uint32_t w = xr[(size_t)hh * half];
    const float e = __uint_as_float(w << 16), o = __uint_as_float(w & 0xffff0000u);
    orow[(size_t)hh * half] = pack_bf16x2(fmaf(e, cs, -o * sn), fmaf(e, sn, o * cs));
  }
}

template <int G>
static void launch_attn_g(const AttnParams& p, bool ks, hipStream_t s) {
  constexpr int PPW = AT_NQ * (16 / G);
  if (ks) {
    const dim3 grid((p.Tq + PPW - 1) / PPW, p.Hkv, p.B);
    hipLaunchKernelGGL((attn_kernel<G, true>), grid, dim3(AttnShape<true>::NW * 64), 0, s, p);
  } else {
    constexpr int QB = AttnShape<false>::NW * PPW;
    const dim3 grid((p.Tq + QB - 1) / QB, p.Hkv, p.B);
    hipLaunchKernelGGL((attn_kernel<G, false>), grid, dim3(AttnShape<false>::NW * 64), 0, s, p);
  }
}

int attn_positions_per_wave(int G) { return AT_NQ * (16 / G); }

int launch_attention(const AttnParams& p, hipStream_t s) {
  const int G = p.Hq / p.Hkv;
  // the key split when one wave holds every position of a sequence (as in
  // decode): the query split would leave three waves idle
  const bool ks = p.Tq <= attn_positions_per_wave(G);
  switch (G) {
    case 1: launch_attn_g<1>(p, ks, s); break;
    case 2: launch_attn_g<2>(p, ks, s); break;
    case 4: launch_attn_g<4>(p, ks, s); break;
    case 8: launch_attn_g<8>(p, ks, s); break;
    case 16: launch_attn_g<16>(p, ks, s); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_rope(const uint16_t* x, uint16_t* out, int n, int H, int D, int pos0, float theta, hipStream_t s) {
  const long long threads = (long long)n * (D / 2);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(rope_kernel, dim3(blocks), dim3(256), 0, s, x, out, n, H, D, pos0, log2((double)theta));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
