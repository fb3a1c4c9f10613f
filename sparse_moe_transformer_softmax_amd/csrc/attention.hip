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
//   O^T += V^T P^T   A = 16 head elements x 32 keys from a transposed copy of
//                    the value tile in LDS, B = P^T straight from the softmax's
//                    registers (the MFMA's K order is chosen to match them).
//                    P is fed as two bf16 terms, hi = bf16(p) and
//                    lo = bf16(p - hi), so the products carry p to about 2^-17.
// The output O^T has the same one-column-per-lane layout as the softmax
// state, so rescaling needs no data movement.
//
// Two launch shapes:
//   query split (KS = false): the four waves own 4 * NQ blocks of columns and
//     share every key/value tile, which the workgroup stages in LDS (double
//     buffered, one barrier per tile);
//   key split (KS = true, a workgroup's positions fit one wave, as in decode):
//     the four waves own the same columns and take every fourth tile each,
//     each staging its own tiles; their partial states are merged at the end
//     in wave order, so the result does not depend on timing.
#include "moe_common.h"
#include "moe_kernels.h"

#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "attention.hip is written for gfx950 only"
#endif

namespace moe {

constexpr int AT_D = 64;              // head width
constexpr int AT_BK = 32;             // keys per tile
constexpr int AT_NW = 4;              // waves per workgroup
constexpr int AT_NQ = 2;              // 16-column blocks per wave
constexpr int AT_TILE_BYTES = AT_BK * AT_D * 2;  // 4 KB of keys or of values

// LDS copy of one tile: keys as rows of 128 bytes whose 16-byte chunks are
// XOR-swizzled by the key's low three bits; values transposed, one row of 64
// bytes per head element whose 8-byte chunks (four keys each) are swizzled by
// bits 1..3 of the element index.  Both make the MFMA operand reads free of
// bank conflicts.
struct AttnTile {
  uint8_t k[AT_TILE_BYTES];
  uint8_t vt[AT_TILE_BYTES];
};

__device__ __forceinline__ uint32_t k_lds_off(int key, int chunk) { return key * 128 + ((chunk ^ (key & 7)) << 4); }
__device__ __forceinline__ uint32_t vt_lds_off(int d, int key) {
  return d * 64 + (((key >> 2) ^ ((d >> 1) & 7)) << 3) + ((key & 3) << 1);
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
    const uint32_t w[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *(uint16_t*)(s.vt + vt_lds_off(8 * c + e, key)) = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// Running softmax state of the lane's NQ query columns and their O^T blocks
// (head elements 16 db + 4 g .. + 3 of column r of block n in acc[n][db]).
struct AttnState {
  float m[AT_NQ], l[AT_NQ];
  v4f acc[AT_NQ][AT_D / 16];
};

// One tile for the lane's NQ column blocks.  pos[n] is the position of the
// lane's column in block n (any value for columns past the batch: their keys
// are all masked).
__device__ __forceinline__ void attn_tile(const AttnTile& s, int t, const v8bf (&qf)[AT_NQ][2],
                                          const int (&pos)[AT_NQ], const bool (&live)[AT_NQ], int window,
                                          float scale, AttnState& st) {
  const int lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
  // K fragments: key 16 kb + r, head elements 32 ks + 8 g .. + 7
  v8bf kf[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      kf[kb][ks] = *(const v8bf*)(s.k + k_lds_off(16 * kb + r, 4 * ks + g));
  // V^T fragments: head element 16 db + r, keys 4g .. 4g+3 and 16+4g .. 16+4g+3
  v8bf vf[AT_D / 16];
#pragma unroll
  for (int db = 0; db < AT_D / 16; ++db) {
    const int d = 16 * db + r;
    const uint2 a = *(const uint2*)(s.vt + vt_lds_off(d, 4 * g));
    const uint2 c = *(const uint2*)(s.vt + vt_lds_off(d, 16 + 4 * g));
    const uint4 w = make_uint4(a.x, a.y, c.x, c.y);
    vf[db] = __builtin_bit_cast(v8bf, w);
  }
#pragma unroll
  for (int n = 0; n < AT_NQ; ++n) {
    v4f sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sc[kb] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][ks], qf[n][ks], sc[kb], 0, 0, 0);
    }
    // mask and scale; key of sc[kb][e] is 32 t + 16 kb + 4 g + e
    float x[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = AT_BK * t + 16 * kb + 4 * g + e;
        const bool ok = live[n] && key <= pos[n] && (window == 0 || pos[n] - key < window);
        const float v = ok ? sc[kb][e] * scale : -INFINITY;
        x[4 * kb + e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(st.m[n], mx);
    const bool none = mnew == -INFINITY;  // no key and no finite sink yet
    const float alpha = none ? 1.f : exp2f(st.m[n] - mnew);
    float ps = 0.f;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float p0 = none ? 0.f : exp2f(x[e] - mnew), p1 = none ? 0.f : exp2f(x[e + 1] - mnew);
      ps += p0 + p1;
      const uint32_t h = pack_bf16x2(p0, p1);
      hi[e >> 1] = h;
      lo[e >> 1] = pack_bf16x2(p0 - __uint_as_float(h << 16), p1 - __uint_as_float(h & 0xffff0000u));
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    st.l[n] = st.l[n] * alpha + ps;
    st.m[n] = mnew;
    const v8bf phi = __builtin_bit_cast(v8bf, make_uint4(hi[0], hi[1], hi[2], hi[3]));
    const v8bf plo = __builtin_bit_cast(v8bf, make_uint4(lo[0], lo[1], lo[2], lo[3]));
#pragma unroll
    for (int db = 0; db < AT_D / 16; ++db) {
      v4f a = st.acc[n][db] * alpha;
      a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], phi, a, 0, 0, 0);
      st.acc[n][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], plo, a, 0, 0, 0);
    }
  }
}

template <int G, bool KS>
__global__ __launch_bounds__(AT_NW * 64) void attn_kernel(AttnParams p) {
  constexpr int PPB = 16 / G;            // positions per column block
  constexpr int PPW = AT_NQ * PPB;       // positions per wave
  constexpr int QB = KS ? PPW : AT_NW * PPW;  // positions per workgroup
  constexpr int MRG = 2 * AT_NQ + AT_NQ * AT_D / 4;  // m, l and O^T of a lane's columns
  __shared__ AttnTile s_tile[KS ? AT_NW : 2];
  __shared__ float s_merge[KS ? AT_NW : 1][KS ? 64 : 1][KS ? MRG : 1];

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
#pragma unroll
  for (int n = 0; n < AT_NQ; ++n) {
    qi[n] = i0 + (KS ? 0 : wave * PPW) + n * PPB + r / G;
    live[n] = qi[n] < p.Tq;
    pos[n] = p.q_pos0 + qi[n];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (live[n]) w = *(const uint4*)(p.q + (((size_t)b * p.Tq + qi[n]) * p.Hq + h) * AT_D + 32 * ks + 8 * g);
      qf[n][ks] = __builtin_bit_cast(v8bf, w);
    }
  }
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

  if constexpr (!KS) {
    // query split: 256 threads stage each tile, one chunk of keys and one of
    // values each; the next tile's loads are in flight during this tile
    TileRegs<1> rg;
    tile_load<1>(p, b, hk, t0, tid, AT_NW * 64, rg);
    for (int t = t0; t <= t1; ++t) {
      AttnTile& s = s_tile[(t - t0) & 1];
      tile_store<1>(s, tid, AT_NW * 64, rg);
      __syncthreads();  // tile t staged; every wave is done with tile t - 2's buffer
      if (t < t1) tile_load<1>(p, b, hk, t + 1, tid, AT_NW * 64, rg);
      attn_tile(s, t, qf, pos, live, p.window, p.qk_scale, st);
    }
  } else {
    // key split: wave w takes tiles t0 + w, t0 + w + 4, ..., staging each in
    // its own LDS tile (64 lanes, four chunks of keys and four of values each)
    AttnTile& s = s_tile[wave];
    TileRegs<4> rg;
    int t = t0 + wave;
    if (t <= t1) tile_load<4>(p, b, hk, t, lane, 64, rg);
    for (; t <= t1; t += AT_NW) {
      tile_store<4>(s, lane, 64, rg);
      if (t + AT_NW <= t1) tile_load<4>(p, b, hk, t + AT_NW, lane, 64, rg);
      attn_tile(s, t, qf, pos, live, p.window, p.qk_scale, st);
    }
    // merge the four waves' states in wave order
    float* mine = &s_merge[wave][lane][0];
#pragma unroll
    for (int n = 0; n < AT_NQ; ++n) {
      mine[0 + n] = st.m[n];
      mine[AT_NQ + n] = st.l[n];
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) mine[2 * AT_NQ + (n * (AT_D / 16) + db) * 4 + e] = st.acc[n][db][e];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int n = 0; n < AT_NQ; ++n) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < AT_NW; ++w) M = fmaxf(M, s_merge[w][lane][n]);
      float L = 0.f;
      v4f O[AT_D / 16];
#pragma unroll
      for (int db = 0; db < AT_D / 16; ++db) O[db] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < AT_NW; ++w) {
        const float mw = s_merge[w][lane][n];
        const float f = (M == -INFINITY || mw == -INFINITY) ? 0.f : exp2f(mw - M);
        L += s_merge[w][lane][AT_NQ + n] * f;
#pragma unroll
        for (int db = 0; db < AT_D / 16; ++db)
#pragma unroll
          for (int e = 0; e < 4; ++e) O[db][e] += s_merge[w][lane][2 * AT_NQ + (n * (AT_D / 16) + db) * 4 + e] * f;
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
    hipLaunchKernelGGL((attn_kernel<G, true>), grid, dim3(AT_NW * 64), 0, s, p);
  } else {
    const dim3 grid((p.Tq + AT_NW * PPW - 1) / (AT_NW * PPW), p.Hkv, p.B);
    hipLaunchKernelGGL((attn_kernel<G, false>), grid, dim3(AT_NW * 64), 0, s, p);
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
