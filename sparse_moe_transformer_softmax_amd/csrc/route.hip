// Router GEMM fused with top-k selection, the selected-expert softmax, the
// per-expert row lists and the MX6x3 split of the token rows.
//
// Method steps (gpt-oss pages): a router scores every expert for each token
// ("【LLM】GPT-OSS架构变化详解", 2.4.1 MoE 的核心原理); each token keeps its
// top-4 experts and weights them by a softmax over the selected logits
// ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", 模型架构: MoE item).
//
// One workgroup (4 waves) owns 16*MBR consecutive tokens and all E experts:
//  1. logits = x W_r^T with v_mfma_f32_16x16x32_bf16 (bf16 products are exact
//     in fp32, fp32 accumulation), plus the fp32 bias;
//  2. per token, k rounds of a wave-wide arg-max (ties -> lower expert id),
//     softmax over the k selected logits;
//  3. per expert, a 64-bit token mask in LDS gives every (token, slot) pair a
//     stable rank inside the workgroup; one atomic per (workgroup, expert)
//     reserves the workgroup's slice of that expert's row list;
//  4. the workgroup's token rows are split into MX6x3 operand rows for the
//     gate/up GEMM;
//  5. the last workgroup to finish (release/acquire through a device-scope
//     counter) turns the per-expert counts into offsets and the GEMM tile
//     list, then clears the counters for the next call.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

constexpr int RT_THREADS = 256;
constexpr int RT_MAXCB = 4;  // 16-expert column blocks per wave (E <= 256)

template <int MBR>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteParams p) {
  constexpr int MT = 16 * MBR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * MT;
  const int T = p.T, d = p.d, E = p.E, k = p.k;
  const int ncb = (E + 15) >> 4;

  __shared__ float s_logit[MT][257];
  __shared__ unsigned long long s_mask[256];
  __shared__ int s_base[256];
  __shared__ int s_ids[MT * 8];
  __shared__ int s_scan[256];
  __shared__ int s_flag;

  for (int e = tid; e < 256; e += RT_THREADS) s_mask[e] = 0ull;

  // ---- 1. router GEMM -------------------------------------------------
  {
    const int g = lane >> 4, r = lane & 15;
    v4f acc[MBR][RT_MAXCB];
#pragma unroll
    for (int i = 0; i < MBR; ++i)
#pragma unroll
      for (int j = 0; j < RT_MAXCB; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
    const uint16_t* xrow[MBR];
    bool xok[MBR];
#pragma unroll
    for (int i = 0; i < MBR; ++i) {
      const int t = t0 + 16 * i + r;
      xok[i] = t < T;
      xrow[i] = p.x + (size_t)(xok[i] ? t : 0) * d + 8 * g;
    }
    const uint16_t* wrow[RT_MAXCB];
    bool wok[RT_MAXCB];
#pragma unroll
    for (int j = 0; j < RT_MAXCB; ++j) {
      const int cb = wave + 4 * j;
      const int e = cb * 16 + r;
      wok[j] = (cb < ncb) && (e < E);
      wrow[j] = p.router_w + (size_t)(wok[j] ? e : 0) * d + 8 * g;
    }
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    for (int kk = 0; kk < d; kk += 32) {
      uint4 a[MBR], b[RT_MAXCB];
#pragma unroll
      for (int i = 0; i < MBR; ++i) a[i] = xok[i] ? *(const uint4*)(xrow[i] + kk) : zero4;
#pragma unroll
      for (int j = 0; j < RT_MAXCB; ++j) b[j] = wok[j] ? *(const uint4*)(wrow[j] + kk) : zero4;
#pragma unroll
      for (int j = 0; j < RT_MAXCB; ++j) {
        if (wave + 4 * j >= ncb) continue;
#pragma unroll
        for (int i = 0; i < MBR; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[i]),
                                                             __builtin_bit_cast(v8bf, b[j]), acc[i][j], 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < RT_MAXCB; ++j) {
      const int cb = wave + 4 * j;
      if (cb >= ncb) continue;
      const int e = cb * 16 + (lane & 15);
      const float bias = e < E ? p.router_b[e] : 0.f;
#pragma unroll
      for (int i = 0; i < MBR; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) s_logit[16 * i + 4 * (lane >> 4) + q][e] = acc[i][j][q] + bias;
    }
  }
  __syncthreads();

  // ---- 2. top-k + softmax ------------------------------------------------
  for (int tl = wave; tl < MT; tl += 4) {
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
    float sel_v[8];
    int sel_e[8];
    for (int j = 0; j < k; ++j) {
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
      sel_v[j] = bv;
      sel_e[j] = be;
    }
    // the raw logit (NaN included) decides the weight
    const float m = sel_v[0];
    float den = 0.f;
    for (int j = 0; j < k; ++j) den += expf(sel_v[j] - m);
    if (lane < k) {
      float myv = sel_v[0];
      int mye = sel_e[0];
      for (int j = 1; j < k; ++j)
        if (lane == j) { myv = sel_v[j]; mye = sel_e[j]; }
      const float raw = s_logit[tl][mye];
      const float w = (raw != raw) ? raw : expf(myv - m) / den;
      p.topk_id[(size_t)t * k + lane] = mye;
      p.topk_w[(size_t)t * k + lane] = w;
      s_ids[tl * k + lane] = mye;
      atomicOr(&s_mask[mye], 1ull << tl);
    }
  }
  __syncthreads();

  // ---- 3. per-expert row lists ---------------------------------------------
  for (int e = tid; e < E; e += RT_THREADS) {
    const int c = __popcll(s_mask[e]);
    s_base[e] = c ? atomicAdd(&p.cursor[e], c) : 0;
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

  // ---- 4. MX6x3 split of the token rows -------------------------------------
  {
    const int nblk = d >> 5;
    for (int u = tid; u < ntok * nblk; u += RT_THREADS) {
      const int tl = u / nblk, b = u - tl * nblk;
      const uint16_t* src = p.x + (size_t)(t0 + tl) * d + 32 * b;
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 w4 = ((const uint4*)src)[q];
        const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[8 * q + 2 * h] = __uint_as_float(ws[h] << 16);
          v[8 * q + 2 * h + 1] = __uint_as_float(ws[h] & 0xffff0000u);
        }
      }
      uint8_t codes[3][32];
      int sc[3];
      mx6x3_split(v, codes, sc);
      uint32_t* dst = (uint32_t*)(p.xq + ((size_t)(t0 + tl) * nblk + b) * MX6_BLOCK_BYTES);
      uint32_t pk[6];
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        pack6x32(codes[t], pk);
        uint2* d2 = (uint2*)(dst + 6 * t);
        d2[0] = make_uint2(pk[0], pk[1]);
        d2[1] = make_uint2(pk[2], pk[3]);
        d2[2] = make_uint2(pk[4], pk[5]);
      }
      ((uint2*)dst)[9] = make_uint2((uint32_t)sc[0] | ((uint32_t)sc[1] << 8) | ((uint32_t)sc[2] << 16), 0u);
    }
  }

  // ---- 5. last workgroup: offsets, tile list, counter reset ----------------
  __threadfence();
  __syncthreads();
  if (tid == 0) s_flag = (atomicAdd(p.done, 1) == (int)gridDim.x - 1);
  __syncthreads();
  if (!s_flag) return;
  __threadfence();
  const int e = tid;
  int cnt = 0, nt = 0;
  if (e < E) {
    cnt = atomicAdd(&p.cursor[e], 0);
    nt = (cnt + p.mt - 1) / p.mt;
    p.counts[e] = cnt;
  }
  // inclusive scans over E (<= 256) of cnt and nt, packed in one int each pass
  int vals[2] = {cnt, nt};
  int incl[2];
  for (int s = 0; s < 2; ++s) {
    s_scan[tid] = vals[s];
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    incl[s] = s_scan[tid];
    __syncthreads();
  }
  if (e < E) {
    p.offsets[e] = incl[0] - cnt;
    const int tb = incl[1] - nt;
    for (int i = 0; i < nt; ++i) p.tiles[tb + i] = make_int2(e, i * p.mt);
    p.cursor[e] = 0;
    if (e == E - 1) {
      p.offsets[E] = incl[0];
      *p.n_tiles = incl[1];
    }
  }
  if (tid == 0) *p.done = 0;
}

int launch_route(const RouteParams& p, hipStream_t stream) {
  if (p.T <= 1024) {
    const int grid = (p.T + 15) / 16;
    hipLaunchKernelGGL(route_kernel<1>, dim3(grid), dim3(RT_THREADS), 0, stream, p);
  } else {
    const int grid = (p.T + 31) / 32;
    hipLaunchKernelGGL(route_kernel<2>, dim3(grid), dim3(RT_THREADS), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
