// Router GEMM fused with top-k selection, the selected-expert softmax, the
// per-expert row lists and the GEMM tile list; trailing workgroups of the
// same launch write the MX6x3 split of the token rows.
//
// Method steps (gpt-oss pages): a router scores every expert for each token
// ("【LLM】GPT-OSS架构变化详解", 2.4.1 MoE 的核心原理); each token keeps its
// top-4 experts and weights them by a softmax over the selected logits
// ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", 模型架构: MoE item).
//
// A token block of MT = 16*MBR consecutive tokens is handled by ks
// workgroups (16 waves each) that split K; every workgroup sees all E
// experts:
//  1. logits = x W_r^T with v_mfma_f32_16x16x32_bf16 (bf16 products are exact
//     in fp32, fp32 accumulation).  The waves split the workgroup's K range
//     and the expert column blocks; partials are summed in a fixed order
//     (waves in LDS, then workgroups: the last workgroup of the block to
//     finish adds the others' partials, exchanged through memory), plus the
//     fp32 bias;
//  2. per token, the k largest logits (ties -> lower expert id): for
//     E <= 64 each expert's rank among all E logits (ranks below k are the
//     slots), for larger E k rounds of a wave-wide arg-max; then the softmax
//     over the k selected logits;
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

__device__ __forceinline__ void lds_wave_sync_route() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
constexpr int RT_LS = 260;        // LDS row stride of the logits (16-byte aligned rows)

// MX6x3 split of one 32-element block of x by four lanes (q4 = lane % 4
// holds elements 8q4 .. 8q4+7): the activation operand of the gate/up GEMM,
// written in the piece-interleaved row layout.
__device__ __forceinline__ void split_block(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, int u, int nblk,
                                            int d, int q4, bool ok) {
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
  uint8_t* row = xq + (size_t)t * mx6_row_bytes(nblk);
  // 2-byte stores never straddle a 16-byte piece (even offsets)
#pragma unroll
  for (int tt = 0; tt < 3; ++tt)
#pragma unroll
    for (int h = 0; h < 3; ++h)
      *(uint16_t*)(row + mx6_byte_offset(b, 24 * tt + 6 * q4 + 2 * h)) = (uint16_t)(bits[tt] >> (16 * h));
  if (q4 == 0)
    *(uint2*)(row + mx6_byte_offset(b, 72)) =
        make_uint2((uint32_t)sc[0] | ((uint32_t)sc[1] << 8) | ((uint32_t)sc[2] << 16), 0u);
}

// NCBW: 16-expert column blocks per wave (1 for E <= 64, 2 for E <= 128,
// 4 for E <= 256); MBR: 16-token row blocks per workgroup (2 only with
// E <= 128, to bound the LDS partials)
// EPL: experts per lane in the top-k ranking (ceil(E / 64))
template <int NCBW, int MBR, int EPL>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteParams p) {
  constexpr int MT = 16 * MBR;
  // K steps in flight (<= 18 b128 loads; fewer at NCBW = 4 to stay within 128 VGPRs)
  constexpr int BATCH = NCBW >= 4 ? 2 : ((18 / (MBR + NCBW)) > 2 ? 18 / (MBR + NCBW) : 2);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, d = p.d, E = p.E, k = p.k;
  const int nblk = d >> 5;

  // ---- trailing workgroups: MX6x3 split of x (256 blocks each) ----------
  const int nrw = p.n_tb * p.ks;
  if ((int)blockIdx.x >= nrw) {
    const int u = ((int)blockIdx.x - nrw) * (RT_THREADS / 4) + (tid >> 2);
    split_block(p.x, p.xq, u, nblk, d, tid & 3, u < T * nblk);
    return;
  }

  const int tb = blockIdx.x / p.ks, kslice = blockIdx.x - tb * p.ks;
  const int t0 = tb * MT;
  const int ncb = (E + 15) >> 4;
  // this workgroup's K blocks; its waves = KS K-sub-slices x EG expert
  // groups, a wave owning column blocks eg, eg + EG, ... of its sub-slice
  const int kb0 = kslice * nblk / p.ks, kb1 = (kslice + 1) * nblk / p.ks;
  const int EG = (ncb + NCBW - 1) / NCBW;
  const int KS = 16 / EG;
  const int eg = wave % EG, ks = wave / EG;  // waves with ks >= KS idle in the GEMM
  const int ES = 16 * ncb + 1;               // row stride of the partials

  __shared__ float s_part[16 * 1032];        // [KS][MT][ES]: KS * MT * ES <= 16 * 1032
  __shared__ __align__(16) float s_logit[MT][RT_LS];
  __shared__ unsigned long long s_mask[256];
  __shared__ int s_base[256];
  __shared__ int s_ids[MT * 8];
  __shared__ float s_ex[MT][8];
  __shared__ int s_scan[256];
  __shared__ int s_flag;

  for (int e = tid; e < 256; e += RT_THREADS) s_mask[e] = 0ull;

  // ---- 1. router GEMM over K blocks [kb0, kb1) ---------------------------
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
    const int s0 = kb0 + ks * (kb1 - kb0) / KS, s1 = kb0 + (ks + 1) * (kb1 - kb0) / KS;
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
  // fixed-order sum over the waves' sub-slices
  for (int u = tid; u < MT * E; u += RT_THREADS) {
    const int tl = u / E, e = u - tl * E;
    float v = 0.f;
    for (int q = 0; q < KS; ++q) v += s_part[(q * MT + tl) * ES + e];
    s_logit[tl][e] = v;
  }

  // ---- K-split exchange: every workgroup of the token block writes its
  // partial logits with stores that reach the device-coherent level, waits
  // for them, and counts itself in; the last one sums the partials in slice
  // order (loads from the same level) and carries on alone ----
  if (p.ks > 1) {
    __syncthreads();
    float* part = p.part + (size_t)tb * p.ks * MT * E;
    for (int u = tid; u < MT * E; u += RT_THREADS)
      __hip_atomic_store(part + (size_t)kslice * MT * E + u, s_logit[u / E][u - (u / E) * E], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the partials have reached memory
    __syncthreads();
    if (tid == 0) s_flag = (atomicAdd(p.tb_done + tb * CURSOR_STRIDE, 1) == p.ks - 1);
    __syncthreads();
    if (!s_flag) return;
    for (int u = tid; u < MT * E; u += RT_THREADS) {
      // all slices' loads in flight at once, then the sum in slice order
      float pv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        pv[q] = q < p.ks ? __hip_atomic_load(part + (size_t)q * MT * E + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < p.ks) v += pv[q];
      s_logit[u / E][u - (u / E) * E] = v;
    }
    if (tid == 0) atomicExch(p.tb_done + tb * CURSOR_STRIDE, 0);
  }
  __syncthreads();
  for (int u = tid; u < MT * E; u += RT_THREADS) s_logit[u / E][u - (u / E) * E] += p.router_b[u - (u / E) * E];
  __syncthreads();

  // ---- 2. top-k + softmax: one wave per token -----------------------------
  for (int tl = wave; tl < MT; tl += RT_THREADS / 64) {
    const int t = t0 + tl;
    if (t >= T) break;
    if constexpr (EPL == 1) {
      // E <= 64: each lane ranks its expert against all E logits (ties ->
      // lower id; NaN never wins a slot); rank j < k takes slot j, so slots
      // follow descending logit.  Ordering key: the logit's bits made
      // monotone as an unsigned integer above the complement of the id.
      auto key_of = [](float x, int e) -> uint64_t {
        // NaN -> -inf; -0 -> +0 (equal logits tie on the id)
        const uint32_t b = (x != x) ? 0xff800000u : (x == 0.0f ? 0u : __float_as_uint(x));
        const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
        return ((uint64_t)o << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
      };
      const int e = lane;
      const float x = e < E ? s_logit[tl][e] : -__builtin_inff();
      const float v = (x != x) ? -__builtin_inff() : x;
      const uint64_t key = key_of(x, e);
      int rank = 0;
      float m = -__builtin_inff();
      for (int e4 = 0; e4 < E; e4 += 4) {
        const v4f w4 = *(const v4f*)&s_logit[tl][e4];  // same address on every lane: a broadcast
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int e2 = e4 + c;
          const bool in = e2 < E;
          m = in ? fmaxf(m, (w4[c] != w4[c]) ? -__builtin_inff() : w4[c]) : m;
          rank += (in && key_of(w4[c], e2) > key) ? 1 : 0;
        }
      }
      // softmax over the selected logits: e^(l - max), summed in slot order
      if (e < E && rank < k) {
        s_ex[tl][rank] = expf(v - m);
        s_ids[tl * k + rank] = e;
      }
      lds_wave_sync_route();
      if (lane < k) {
        float den = 0.f;
        for (int j = 0; j < k; ++j) den += s_ex[tl][j];
        const int es = s_ids[tl * k + lane];
        const float raw = s_logit[tl][es];
        p.topk_id[(size_t)t * k + lane] = es;
        p.topk_w[(size_t)t * k + lane] = (raw != raw) ? raw : s_ex[tl][lane] / den;
        atomicOr(&s_mask[es], 1ull << tl);
      }
    } else {
      // E > 64: k rounds of a wave-wide arg-max (ties -> lower id; NaN
      // never wins a slot); lane j keeps the value and id of slot j
      float v[EPL];
      bool taken[EPL];
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        const float x = e < E ? s_logit[tl][e] : -__builtin_inff();
        v[i] = (x != x) ? -__builtin_inff() : x;
        taken[i] = e >= E;
      }
      float my_v = -__builtin_inff(), m = -__builtin_inff();
      int my_e = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j >= k) break;
        float bv = -__builtin_inff();
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
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
        for (int i = 0; i < EPL; ++i)
          if (lane + 64 * i == be) taken[i] = true;
        if (j == 0) m = bv;
        if (lane == j) { my_v = bv; my_e = be; }
      }
      // softmax over the selected logits (the raw logit, NaN included,
      // decides the weight)
      const float ex = (lane < k) ? expf(my_v - m) : 0.f;
      float den = ex;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
      if (lane < k) {
        const float raw = s_logit[tl][my_e];
        p.topk_id[(size_t)t * k + lane] = my_e;
        p.topk_w[(size_t)t * k + lane] = (raw != raw) ? raw : ex / den;
        s_ids[tl * k + lane] = my_e;
        atomicOr(&s_mask[my_e], 1ull << tl);
      }
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

  // ---- 4. last token block: offsets, tile list, counter reset -------------
  if (tid == 0) s_flag = (atomicAdd(p.done, 1) == p.n_tb - 1);
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

// LDS partials of a configuration: KS * MT * ES floats must fit s_part
static bool route_fits(int ncb, int ncbw, int mbr) {
  const int eg = (ncb + ncbw - 1) / ncbw, ks = 16 / eg;
  return ks >= 1 && ks * 16 * mbr * (16 * ncb + 1) <= 16 * 1032;
}

// Workgroups per token block: small batches split K over several
// workgroups so that the router weight streams through more CUs.
int route_kslices(int T, int E) {
  const int ncb = (E + 15) / 16;
  const bool big = T >= 2048 && ncb <= 8;
  const int n_tb = (T + (big ? 31 : 15)) / (big ? 32 : 16);
  if (n_tb >= ROUTE_MAX_SPLIT_BLOCKS) return 1;
  const int ks = ROUTE_MAX_SPLIT_BLOCKS / n_tb;
  return ks < 8 ? ks : 8;
}

int launch_route(const RouteParams& p0, hipStream_t stream) {
  RouteParams p = p0;
  const int ncb = (p.E + 15) / 16;
  const bool big = p.T >= 2048 && ncb <= 8;
  p.n_tb = (p.T + (big ? 31 : 15)) / (big ? 32 : 16);
  p.ks = route_kslices(p.T, p.E);
  const int ncbw = big ? (ncb <= 4 ? 1 : 2) : (ncb <= 8 ? 2 : 4);
  if (!route_fits(ncb, ncbw, big ? 2 : 1)) return -1;
  if (p.ks > 1 && (p.part == nullptr || p.tb_done == nullptr || p.n_tb * p.ks > ROUTE_MAX_SPLIT_BLOCKS)) return -1;
  const long long quads = p.xq ? (long long)p.T * (p.d / 32) : 0;
  const long long grid = (long long)p.n_tb * p.ks + (quads + RT_THREADS / 4 - 1) / (RT_THREADS / 4);
  const dim3 g((unsigned)grid), b(RT_THREADS);
  const int epl = (p.E + 63) / 64;
#define MOE_ROUTE(NCBW, MBR)                                                                      \
  do {                                                                                            \
    if (epl == 1)                                                                                 \
      hipLaunchKernelGGL((route_kernel<NCBW, MBR, 1>), g, b, 0, stream, p);                       \
    else if (epl == 2)                                                                            \
      hipLaunchKernelGGL((route_kernel<NCBW, MBR, 2>), g, b, 0, stream, p);                       \
    else                                                                                          \
      hipLaunchKernelGGL((route_kernel<NCBW, MBR, 4>), g, b, 0, stream, p);                       \
  } while (0)
  if (big) {
    if (ncb <= 4)
      MOE_ROUTE(1, 2);
    else
      MOE_ROUTE(2, 2);
  } else {
    if (ncb <= 8)
      MOE_ROUTE(2, 1);
    else
      MOE_ROUTE(4, 1);
  }
#undef MOE_ROUTE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
