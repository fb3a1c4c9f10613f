// Router GEMM fused with top-k selection, the selected-expert softmax, the
// per-expert row lists and the GEMM tile list; and the MX6x3 split of the
// token rows (a kernel of its own).
//
// Method steps (gpt-oss pages): a router scores every expert for each token
// ("【LLM】GPT-OSS架构变化详解", 2.4.1 MoE 的核心原理); each token keeps its
// top-4 experts and weights them by a softmax over the selected logits
// ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", 模型架构: MoE item).
//
// One workgroup (16 waves) owns MT = 16*MBR consecutive tokens and all E
// experts:
//  1. logits = x W_r^T with v_mfma_f32_16x16x32_bf16 (bf16 products are exact
//     in fp32, fp32 accumulation).  The waves split K and the expert column
//     blocks; the K-slice partials are summed in a fixed order in LDS, plus
//     the fp32 bias;
//  2. per token, k rounds of a wave-wide arg-max (ties -> lower expert id),
//     softmax over the k selected logits;
//  3. per expert, a 64-bit token mask in LDS gives every (token, slot) pair a
//     stable rank inside the workgroup; one returning atomic per
//     (workgroup, expert) reserves the workgroup's slice of that expert's row
//     list;
//  4. the last workgroup to finish (device-scope atomic counter; it reads only
//     atomically updated counters, so no cache-flushing fence is needed)
//     turns the per-expert counts into offsets and the GEMM tile list, then
//     clears the counters for the next call.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int RT_THREADS = 1024;  // 16 waves

// NCBW: 16-expert column blocks per wave (1 for E <= 64, 2 for E <= 128,
// 4 for E <= 256); MBR: 16-token row blocks per workgroup (2 only with
// E <= 128, to bound the LDS partials)
template <int NCBW, int MBR>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteParams p) {
  constexpr int MT = 16 * MBR;
  constexpr int BATCH = (18 / (MBR + NCBW)) > 2 ? 18 / (MBR + NCBW) : 2;  // K steps in flight (<= 18 b128 loads)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * MT;
  const int T = p.T, d = p.d, E = p.E, k = p.k;
  const int ncb = (E + 15) >> 4;
  const int nblk = d >> 5;
  // waves = KS K-slices x EG expert groups; a wave owns column blocks
  // eg, eg + EG, ... of its K-slice
  const int EG = (ncb + NCBW - 1) / NCBW;
  const int KS = 16 / EG;
  const int eg = wave % EG, ks = wave / EG;  // waves with ks >= KS idle in the GEMM
  const int ES = 16 * ncb + 1;               // row stride of the partials

  __shared__ float s_part[16 * 1032];        // [KS][MT][ES]: KS * MT * ES <= 16 * 1032
  __shared__ float s_logit[MT][257];
  __shared__ unsigned long long s_mask[256];
  __shared__ int s_base[256];
  __shared__ int s_ids[MT * 8];
  __shared__ int s_scan[256];
  __shared__ int s_flag;

  for (int e = tid; e < 256; e += RT_THREADS) s_mask[e] = 0ull;

  // ---- 1. router GEMM (+ MX6x3 split of x by expert group 0) --------------
  if (ks < KS) {
    const int g = lane >> 4, r = lane & 15;
    v4f acc[MBR][NCBW];
#pragma unroll
    for (int i = 0; i < MBR; ++i)
#pragma unroll
      for (int j = 0; j < NCBW; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    // rows past T and experts past E read row 0 (their logits are never
    // used), so every load is unconditional
    const uint16_t* xrow[MBR];
#pragma unroll
    for (int i = 0; i < MBR; ++i) {
      const int t = t0 + 16 * i + r;
      xrow[i] = p.x + (size_t)(t < T ? t : 0) * d + 8 * g;
    }
    const uint16_t* wrow[NCBW];
    bool cbok[NCBW];
#pragma unroll
    for (int j = 0; j < NCBW; ++j) {
      const int cb = eg + EG * j;
      const int e = cb * 16 + r;
      cbok[j] = cb < ncb;
      wrow[j] = p.router_w + (size_t)(e < E ? e : 0) * d + 8 * g;
    }
    const int s0 = ks * nblk / KS, s1 = (ks + 1) * nblk / KS;
    for (int sb = s0; sb < s1; sb += BATCH) {
      uint4 a[BATCH][MBR], b[BATCH][NCBW];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const int kk = min(sb + u, s1 - 1) * 32;
#pragma unroll
        for (int i = 0; i < MBR; ++i) a[u][i] = *(const uint4*)(xrow[i] + kk);
#pragma unroll
        for (int j = 0; j < NCBW; ++j) b[u][j] = *(const uint4*)(wrow[j] + kk);
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        if (sb + u >= s1) break;
#pragma unroll
        for (int j = 0; j < NCBW; ++j)
          if (cbok[j])
#pragma unroll
            for (int i = 0; i < MBR; ++i)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u][i]),
                                                                 __builtin_bit_cast(v8bf, b[u][j]), acc[i][j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < NCBW; ++j) {
      if (!cbok[j]) continue;
      const int e = (eg + EG * j) * 16 + r;
#pragma unroll
      for (int i = 0; i < MBR; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) s_part[(ks * MT + 16 * i + 4 * g + q) * ES + e] = acc[i][j][q];
    }
  }
  __syncthreads();
  // fixed-order sum over the K-slices, plus the bias
  for (int u = tid; u < MT * E; u += RT_THREADS) {
    const int tl = u / E, e = u - tl * E;
    float v = 0.f;
    for (int q = 0; q < KS; ++q) v += s_part[(q * MT + tl) * ES + e];
    s_logit[tl][e] = v + p.router_b[e];
  }
  __syncthreads();

  // ---- 2. top-k + softmax ------------------------------------------------
  for (int tl = wave; tl < MT; tl += RT_THREADS / 64) {
    const int t = t0 + tl;
    if (t >= T) break;
    float v[4];
    bool taken[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      float x = e < E ? s_logit[tl][e] : -__builtin_inff();
      v[i] = (x != x) ? -__builtin_inff() : x;  // NaN never wins a slot
      taken[i] = e >= E;
    }
    // k rounds of arg-max; lane j keeps the value and id of slot j
    float my_v = -__builtin_inff(), m = -__builtin_inff();
    int my_e = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      float bv = -__builtin_inff();
      int be = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (!taken[i] && (v[i] > bv || (v[i] == bv && e < be))) { bv = v[i]; be = e; }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oe = __shfl_xor(be, off);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i == be) taken[i] = true;
      if (j == 0) m = bv;
      if (lane == j) { my_v = bv; my_e = be; }
    }
    // softmax over the selected logits (the raw logit, NaN included, decides
    // the weight)
    const float ex = (lane < k) ? expf(my_v - m) : 0.f;
    float den = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
    if (lane < k) {
      const float raw = s_logit[tl][my_e];
      const float w = (raw != raw) ? raw : ex / den;
      p.topk_id[(size_t)t * k + lane] = my_e;
      p.topk_w[(size_t)t * k + lane] = w;
      s_ids[tl * k + lane] = my_e;
      atomicOr(&s_mask[my_e], 1ull << tl);
    }
  }
  __syncthreads();

  // ---- 3. per-expert row lists ---------------------------------------------
  // atomicAdd returns, so each reservation is performed before the barrier
  for (int e = tid; e < E; e += RT_THREADS) {
    const int c = __popcll(s_mask[e]);
    s_base[e] = c ? atomicAdd(&p.cursor[e * CURSOR_STRIDE], c) : 0;
  }
  __syncthreads();
  const int ntok = min(MT, T - t0);
  for (int q = tid; q < ntok * k; q += RT_THREADS) {
    const int tl = q / k, j = q - tl * k;
    const int e = s_ids[q];
    const int rel = s_base[e] + __popcll(s_mask[e] & ((1ull << tl) - 1ull));
    const int pair = (t0 + tl) * k + j;
    p.expert_rows[(size_t)e * T + rel] = pair;
    p.rel_pos[pair] = rel;
  }

  // ---- 4. last workgroup: offsets, tile list, counter reset ----------------
  if (tid == 0) s_flag = (atomicAdd(p.done, 1) == (int)gridDim.x - 1);
  __syncthreads();
  if (!s_flag) return;
  const int e = tid;
  int cnt = 0, nt = 0;
  if (e < E) {
    cnt = atomicAdd(&p.cursor[e * CURSOR_STRIDE], 0);
    nt = (cnt + p.mt - 1) / p.mt;
    p.counts[e] = cnt;
  }
  // inclusive scans over E (<= 256) of cnt and nt
  const int vals[2] = {cnt, nt};
  int incl[2];
  for (int s = 0; s < 2; ++s) {
    if (tid < 256) s_scan[tid] = vals[s];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = (tid < 256 && tid >= off) ? s_scan[tid - off] : 0;
      __syncthreads();
      if (tid < 256) s_scan[tid] += add;
      __syncthreads();
    }
    incl[s] = tid < 256 ? s_scan[tid] : 0;
    __syncthreads();
  }
  if (e < E) {
    p.offsets[e] = incl[0] - cnt;
    const int tb = incl[1] - nt;
    for (int i = 0; i < nt; ++i) p.tiles[tb + i] = make_int2(e, i * p.mt);
    atomicExch(&p.cursor[e * CURSOR_STRIDE], 0);
    if (e == E - 1) {
      p.offsets[E] = incl[0];
      *p.n_tiles = incl[1];
    }
  }
  if (tid == 0) atomicExch(p.done, 0);
}

// MX6x3 split of the token rows: four lanes per 32-element block, one pass
// over x with every lane independent (no loop-carried memory chain).
__global__ __launch_bounds__(256) void split_x_kernel(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq,
                                                      int T, int d) {
  const int nblk = d >> 5;
  const int u = blockIdx.x * 64 + (threadIdx.x >> 2), q4 = threadIdx.x & 3;
  const bool ok = u < T * nblk;
  const int uu = ok ? u : 0;  // out-of-range quads compute on block 0 and store nothing
  const int t = uu / nblk, b = uu - t * nblk;
  const uint4 w4 = *(const uint4*)(x + (size_t)t * d + 32 * b + 8 * q4);
  const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
  float v[8];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    v[2 * h] = __uint_as_float(ws[h] << 16);
    v[2 * h + 1] = __uint_as_float(ws[h] & 0xffff0000u);
  }
  uint64_t bits[3];
  int sc[3];
  mx6x3_split_quad<1, 2>(v, bits, sc);
  if (!ok) return;
  uint8_t* dst = xq + (size_t)uu * MX6_BLOCK_BYTES;
#pragma unroll
  for (int tt = 0; tt < 3; ++tt) {
    uint16_t* d16 = (uint16_t*)(dst + 24 * tt + 6 * q4);
    d16[0] = (uint16_t)bits[tt];
    d16[1] = (uint16_t)(bits[tt] >> 16);
    d16[2] = (uint16_t)(bits[tt] >> 32);
  }
  if (q4 == 0)
    *(uint2*)(dst + 72) = make_uint2((uint32_t)sc[0] | ((uint32_t)sc[1] << 8) | ((uint32_t)sc[2] << 16), 0u);
}

int launch_split_x(const uint16_t* x, uint8_t* xq, int T, int d, hipStream_t stream) {
  const long long quads = (long long)T * (d / 32);
  hipLaunchKernelGGL(split_x_kernel, dim3((unsigned)((quads + 63) / 64)), dim3(256), 0, stream, x, xq, T, d);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// LDS partials of a configuration: KS * MT * ES floats must fit s_part
static bool route_fits(int ncb, int ncbw, int mbr) {
  const int eg = (ncb + ncbw - 1) / ncbw, ks = 16 / eg;
  return ks >= 1 && ks * 16 * mbr * (16 * ncb + 1) <= 16 * 1032;
}

int launch_route(const RouteParams& p, hipStream_t stream) {
  const int ncb = (p.E + 15) / 16;
  const bool big = p.T >= 2048 && ncb <= 8;
  const int grid = (p.T + (big ? 31 : 15)) / (big ? 32 : 16);
  const int ncbw = big ? (ncb <= 4 ? 1 : 2) : (ncb <= 8 ? 2 : 4);
  if (!route_fits(ncb, ncbw, big ? 2 : 1)) return -1;
  if (big) {
    if (ncb <= 4)
      hipLaunchKernelGGL((route_kernel<1, 2>), dim3(grid), dim3(RT_THREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((route_kernel<2, 2>), dim3(grid), dim3(RT_THREADS), 0, stream, p);
  } else {
    if (ncb <= 8)
      hipLaunchKernelGGL((route_kernel<2, 1>), dim3(grid), dim3(RT_THREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((route_kernel<4, 1>), dim3(grid), dim3(RT_THREADS), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
