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
//     stable rank inside the workgroup; with several token blocks one
//     returning atomic per (workgroup, expert) reserves the workgroup's slice
//     of that expert's row list;
//  4. the last token block to finish (device-scope atomic counter; it reads
//     only atomically updated counters, so no cache-flushing fence is
//     needed) turns the per-expert counts into offsets and the GEMM tile
//     list with one wave, then clears the counters for the next call.  A
//     batch that fits one token block (decode) needs neither counter: its
//     counts are the popcounts of the LDS masks.
#include "moe_common.h"
#include "moe_kernels.h"

// The K-split exchange relies on gfx950's cache behaviour for agent-scope
// atomic stores and loads (see the exchange in route_kernel).
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "route.hip is written for gfx950 only"
#endif

namespace moe {

constexpr int RT_THREADS = 1024;  // 16 waves

__device__ __forceinline__ void lds_wave_sync_route() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
constexpr int RT_LS = 260;        // LDS row stride of the logits (16-byte aligned rows)

// MX6x3 split of one 32-element block of x by one lane (block u of the
// token rows, u < T * nblk): the activation operand of the gate/up GEMM,
// written in the piece-interleaved row layout as five 16-byte pieces.  The
// split uses the gfx950 scaled FP6 conversions (round to nearest even with
// the non-saturating block scale), as the split of h does.
__device__ __forceinline__ void split_block(const uint16_t* __restrict__ x, uint8_t* __restrict__ xq, int u, int nblk,
                                            int d) {
  const int t = u / nblk, b = u - t * nblk;
  const uint4* src = (const uint4*)(x + (size_t)t * d + 32 * b);
  v16f ve, vo;  // even and odd elements of the block
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 w = src[i];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      ve[4 * i + h] = __uint_as_float(ws[h] << 16);
      vo[4 * i + h] = __uint_as_float(ws[h] & 0xffff0000u);
    }
  }
  uint32_t codes[18], scw;
  mx6x3_split_lane(ve, vo, codes, scw);
  uint8_t* row = xq + (size_t)t * mx6_row_bytes(nblk);
#pragma unroll
  for (int q = 0; q < 5; ++q) {
    const v4u piece = q < 4 ? (v4u){codes[4 * q], codes[4 * q + 1], codes[4 * q + 2], codes[4 * q + 3]}
                            : (v4u){codes[16], codes[17], scw, 0u};
    *(v4u*)(row + mx6_byte_offset(b, 16 * q)) = piece;
  }
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

  // ---- trailing workgroups: MX6x3 split of x (1024 blocks each) ---------
  const int nrw = p.n_tb * p.ks;
  if ((int)blockIdx.x >= nrw) {
    const int u = ((int)blockIdx.x - nrw) * RT_THREADS + tid;
    // (and clear the arrival counters of the down GEMM's folded combine)
    if (p.fold_cnt)
      for (int i = ((int)blockIdx.x - nrw) * RT_THREADS + tid; i < p.n_fold; i += ((int)gridDim.x - nrw) * RT_THREADS)
        p.fold_cnt[i] = 0;
    if (u < T * nblk) split_block(p.x, p.xq, u, nblk, d);
    return;
  }

  const int tb = blockIdx.x / p.ks, kslice = blockIdx.x - tb * p.ks;
  const int t0 = tb * MT;
  const int ncb = (E + 15) >> 4;
  // this workgroup's K blocks; its waves = KS K-sub-slices x EG expert
  // groups, a wave owning column blocks eg, eg + EG, ... of its sub-slice
  const int kb0 = kslice * nblk / p.ks, kb1 = (kslice + 1) * nblk / p.ks;
  const int EG = (ncb + NCBW - 1) / NCBW;
  const int KS = route_wave_kslices(ncb, NCBW, MBR);
  const int eg = wave % EG, ks = wave / EG;  // waves with ks >= KS idle in the GEMM
  const int ES = 16 * ncb + 1;               // row stride of the partials

  // [KS][MT][ES]: KS * MT * ES <= 16 * 1032; later the top-k keys
  __shared__ __align__(16) float s_part[16 * 1032];
  __shared__ __align__(16) float s_logit[MT][RT_LS];
  __shared__ unsigned long long s_mask[256];
  __shared__ int s_base[256];
  __shared__ int s_ids[MT * 8];
  __shared__ float s_ex[MT][8];
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
    // used); K blocks past the wave's range read beyond the buffer, which
    // returns zeros without memory traffic, so every load and MFMA is
    // unconditional and no load repeats another
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, T * d * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc((void*)p.router_w, 0, E * d * 2, 0x00020000);
    uint32_t xo[MBR], wo[NCBW];
#pragma unroll
    for (int i = 0; i < MBR; ++i) {
      const int t = t0 + 16 * i + r;
      xo[i] = (uint32_t)((t < T ? t : 0) * d + 8 * g) * 2u;
    }
    bool cbok[NCBW];
#pragma unroll
    for (int j = 0; j < NCBW; ++j) {
      const int cb = eg + EG * j;
      const int e = cb * 16 + r;
      cbok[j] = cb < ncb;
      wo[j] = (uint32_t)((e < E ? e : 0) * d + 8 * g) * 2u;
    }
    const int s0 = kb0 + ks * (kb1 - kb0) / KS, s1 = kb0 + (ks + 1) * (kb1 - kb0) / KS;
    // one batch of NB K blocks: every load issued, then the MFMAs
    auto batch = [&](auto nb_c, int sb) {
      constexpr int NB = decltype(nb_c)::value;
      uint4 a[NB][MBR], b[NB][NCBW];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const bool in = sb + u < s1;
        const uint32_t kb = (uint32_t)(sb + u) * 64u;
#pragma unroll
        for (int i = 0; i < MBR; ++i) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, in ? xo[i] + kb : 0xffffff00u, 0, 0);
          a[u][i] = make_uint4(v[0], v[1], v[2], v[3]);
        }
#pragma unroll
        for (int j = 0; j < NCBW; ++j) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(wr, in ? wo[j] + kb : 0xffffff00u, 0, 0);
          b[u][j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // (column blocks past the experts compute on row 0 and are dropped
      // below: a branch here would let the compiler sink the loads into it)
#pragma unroll
      for (int u = 0; u < NB; ++u)
#pragma unroll
        for (int j = 0; j < NCBW; ++j)
#pragma unroll
          for (int i = 0; i < MBR; ++i)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a[u][i]),
                                                               __builtin_bit_cast(v8bf, b[u][j]), acc[i][j], 0, 0, 0);
    };
    // whole batches (the last one partly past the range) while more than two
    // blocks remain, then two at a time: a short K range, as at decode,
    // issues no more loads than it needs (each load instruction costs
    // address-unit time even when it reads nothing), a long one needs no
    // more round trips than full batches
    int sb = s0;
    for (; sb + 2 < s1; sb += BATCH) batch(std::integral_constant<int, BATCH>{}, sb);
    for (; sb < s1; sb += 2) batch(std::integral_constant<int, 2>{}, sb);
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

  if (p.ks == 1) {
    // fixed-order sum over the waves' sub-slices, then the bias
    for (int u = tid; u < MT * E; u += RT_THREADS) {
      const int tl = u / E, e = u - tl * E;
      float v = 0.f;
      for (int q = 0; q < KS; ++q) v += s_part[(q * MT + tl) * ES + e];
      s_logit[tl][e] = v + p.router_b[e];
    }
  } else {
    // ---- K-split exchange: every workgroup of the token block writes its
    // partial logits and counts itself in on the block's arrival counter;
    // the last one sums the partials in slice order, adds the bias and
    // carries on alone.  The workgroups may run on different XCDs, whose
    // L2s are not coherent with each other: the partials go out as
    // device-coherent stores (agent-scope atomic stores, written through to
    // the device-coherent level on gfx950), every wave waits for its stores
    // (vmcnt 0) before the barrier that precedes the arrival, and the last
    // arrival reads them with device-coherent loads issued after it has
    // seen the count.  (An acquire-release arrival orders the same accesses
    // but writes back the XCD's whole L2 per workgroup, which with the x
    // split's rows in flight costs tens of microseconds at prefill sizes.)
    float* part = p.part + (size_t)tb * p.ks * MT * E;
    for (int u = tid; u < MT * E; u += RT_THREADS) {
      const int tl = u / E, e = u - tl * E;
      float v = 0.f;
      for (int q = 0; q < KS; ++q) v += s_part[(q * MT + tl) * ES + e];
      __hip_atomic_store(part + (size_t)kslice * MT * E + u, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_vmcnt<0>();  // this wave's partials are stored
    __syncthreads();
    if (tid == 0)
      s_flag = (__hip_atomic_fetch_add(p.tb_done + tb * CURSOR_STRIDE, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT) == p.ks - 1);
    __syncthreads();
    if (!s_flag) return;
    for (int u = tid; u < MT * E; u += RT_THREADS) {
      // all slices' loads (and the bias) in flight at once, then the sum in
      // slice order
      const float bias = p.router_b[u - (u / E) * E];
      float pv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        pv[q] = q < p.ks ? __hip_atomic_load(part + (size_t)q * MT * E + u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q < p.ks) v += pv[q];
      s_logit[u / E][u - (u / E) * E] = v + bias;
    }
    if (tid == 0) atomicExch(p.tb_done + tb * CURSOR_STRIDE, 0);
  }
  __syncthreads();

  // ---- 2. top-k + softmax --------------------------------------------------
  // Ordering key of a logit: its bits made monotone as an unsigned integer
  // (NaN -> -inf, -0 -> +0, so equal logits tie on the id) above the
  // complement of the expert id; a larger key ranks first.
  auto key_of = [](float x, int e) -> uint64_t {
    const uint32_t b = (x != x) ? 0xff800000u : (x == 0.0f ? 0u : __float_as_uint(x));
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
  };
  const int ntok = min(MT, T - t0);
  if constexpr (EPL == 1) {
    // E <= 64: every (token, expert) pair is one thread's; its rank among the
    // token's E keys (ranks below k are the slots, so slots follow
    // descending logit).  Keys go to LDS once (over the GEMM partials, no
    // longer needed); padding keys are 0, below every real key.
    uint64_t* s_key = (uint64_t*)s_part;  // [MT][64]
    const int EP = (E + 1) & ~1;
    for (int u = tid; u < ntok * 64; u += RT_THREADS) {
      const int tl = u >> 6, e = u & 63;
      if (e < EP) s_key[u] = e < E ? key_of(s_logit[tl][e], e) : 0ull;
    }
    __syncthreads();
    for (int u = tid; u < ntok * E; u += RT_THREADS) {
      const int tl = u / E, e = u - tl * E;
      const uint64_t* kr = s_key + tl * 64;
      const uint64_t key = kr[e];
      int rank = 0;
      for (int e2 = 0; e2 < EP; e2 += 2) {
        const ulonglong2 k2 = *(const ulonglong2*)(kr + e2);
        rank += (k2.x > key) ? 1 : 0;
        rank += (k2.y > key) ? 1 : 0;
      }
      if (rank < k) s_ids[tl * k + rank] = e;
    }
    __syncthreads();
    // softmax over the selected logits: e^(l - max) summed in slot order,
    // max = the slot-0 logit (NaN counted as -inf); a NaN logit's weight is
    // that NaN
    for (int u = tid; u < ntok * k; u += RT_THREADS) {
      const int tl = u / k, j = u - tl * k;
      auto val = [&](int jj) {
        const float x = s_logit[tl][s_ids[tl * k + jj]];
        return (x != x) ? -__builtin_inff() : x;
      };
      const float m = val(0);
      float den = 0.f;
      for (int jj = 0; jj < k; ++jj) den += expf(val(jj) - m);
      const int es = s_ids[tl * k + j];
      const float raw = s_logit[tl][es];
      const int t = t0 + tl;
      p.topk_id[(size_t)t * k + j] = es;
      p.topk_w[(size_t)t * k + j] = (raw != raw) ? raw : expf(val(j) - m) / den;
      atomicOr(&s_mask[es], 1ull << tl);
    }
  } else {
    for (int tl = wave; tl < ntok; tl += RT_THREADS / 64) {
      const int t = t0 + tl;
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
  const bool single = p.n_tb == 1;
  for (int e = tid; e < E; e += RT_THREADS) {
    const int c = __popcll(s_mask[e]);
    s_base[e] = (c && !single) ? atomicAdd(&p.cursor[e * CURSOR_STRIDE], c) : 0;
  }
  __syncthreads();
  for (int q = tid; q < ntok * k; q += RT_THREADS) {
    const int tl = q / k, j = q - tl * k;
    const int e = s_ids[q];
    const int rel = s_base[e] + __popcll(s_mask[e] & ((1ull << tl) - 1ull));
    const int pair = (t0 + tl) * k + j;
    p.expert_rows[(size_t)e * T + rel] = pair;
    p.rel_pos[pair] = rel;
  }

  // ---- 4. last token block: offsets, tile list, counter reset -------------
  if (!single) {
    if (tid == 0) s_flag = (atomicAdd(p.done, 1) == p.n_tb - 1);
    __syncthreads();
    if (!s_flag) return;
  }
  if (wave != 0) return;
  // one wave: lane L owns experts 4L .. 4L+3 (E <= 256); inclusive scans of
  // the counts and tile counts across the lanes
  int c4[4], n4[4], cs = 0, ns = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    c4[i] = e >= E ? 0 : single ? __popcll(s_mask[e]) : atomicAdd(&p.cursor[e * CURSOR_STRIDE], 0);
    n4[i] = (c4[i] + p.mt - 1) / p.mt;
    cs += c4[i];
    ns += n4[i];
  }
  int ci = cs, ni = ns;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ca = __shfl_up(ci, off), na = __shfl_up(ni, off);
    if (lane >= off) { ci += ca; ni += na; }
  }
  int cex = ci - cs, nex = ni - ns;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * lane + i;
    if (e < E) {
      p.counts[e] = c4[i];
      p.offsets[e] = cex;
      for (int j = 0; j < n4[i]; ++j) p.tiles[nex + j] = make_int2(e, j * p.mt);
      if (!single) atomicExch(&p.cursor[e * CURSOR_STRIDE], 0);
    }
    cex += c4[i];
    nex += n4[i];
  }
  if (lane == 63) {
    p.offsets[E] = ci;
    *p.n_tiles = ni;
    if (!single) atomicExch(p.done, 0);
  }
}

// LDS partials of a configuration: KS * MT * ES floats must fit s_part
static bool route_fits(int ncb, int ncbw, int mbr) {
  const int ks = route_wave_kslices(ncb, ncbw, mbr);
  return ks >= 1 && ks * 16 * mbr * (16 * ncb + 1) <= 16 * 1032;
}

// Launch shape of the router: token-block height (16 * mbr), column blocks
// per wave, token blocks and the workgroups per token block.  Every
// workgroup streams the router weight of its K slice, so the K range is
// split over enough workgroups (at most 8 per token block) that about 256
// of them share the weight; batches of 512 tokens or more take 32-token
// blocks; a batch of up to 32 tokens over at most 64 experts is one token
// block.  (Measured at the 20b prefill, 120b Zipf prefill and 120b stack
// sizes against 16- and 64-token blocks and against 512 workgroups: the
// router launch with the x split takes 33, 80 and 39 us; 64-token blocks
// take 35, 101 and 54 us, 16-token blocks 33, 106 and 39 us.)
struct RouteShape {
  int mbr, ncbw, n_tb, ks;
};
static bool route_shape(int T, int E, RouteShape& r) {
  const int ncb = (E + 15) / 16;
  if (T >= 512) {
    r.mbr = 2;
    r.ncbw = ncb <= 4 ? 1 : 2;
  } else {
    const bool one32 = T > 16 && T <= 32 && ncb <= 4 && route_fits(ncb, 1, 2);
    r.mbr = one32 ? 2 : 1;
    r.ncbw = one32 ? 1 : (ncb <= 8 ? 2 : 4);
  }
  r.n_tb = (T + 16 * r.mbr - 1) / (16 * r.mbr);
  r.ks = r.n_tb > ROUTE_MAX_TB ? 1 : (ROUTE_TARGET_WG + r.n_tb - 1) / r.n_tb;
  if (r.ks > 8) r.ks = 8;
  return route_fits(ncb, r.ncbw, r.mbr);
}

size_t route_partial_bytes(int T, int E) {
  RouteShape r;
  if (T <= 0 || !route_shape(T, E, r) || r.ks == 1) return 0;
  return (size_t)r.n_tb * r.ks * 16 * r.mbr * E * sizeof(float);
}

int launch_route(const RouteParams& p0, hipStream_t stream) {
  RouteParams p = p0;
  RouteShape r;
  if (!route_shape(p.T, p.E, r)) return -1;
  p.n_tb = r.n_tb;
  p.ks = r.ks;
  // the partials of all K slices: n_tb * ks * 16 * mbr rows of E floats
  if (p.ks > 1 && (p.part == nullptr || p.tb_done == nullptr || p.n_tb > ROUTE_MAX_TB)) return -1;
  const long long blocks = p.xq ? (long long)p.T * (p.d / 32) : 0;
  const long long grid = (long long)p.n_tb * p.ks + (blocks + RT_THREADS - 1) / RT_THREADS;
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
  if (r.mbr == 2) {
    if (r.ncbw == 1)
      MOE_ROUTE(1, 2);
    else
      MOE_ROUTE(2, 2);
  } else {
    if (r.ncbw == 2)
      MOE_ROUTE(2, 1);
    else
      MOE_ROUTE(4, 1);
  }
#undef MOE_ROUTE
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
