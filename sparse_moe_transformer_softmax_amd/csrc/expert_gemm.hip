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
// Operand layout of the 16x16x128 scaled MFMA (checked by the one-hot
// probe tests): lane l carries row (A) or column (B) l % 16 and the 32
// consecutive K values of block l / 16 of the 128-wide step; the result
// C[4*(l/16) + q][l % 16] sits in accumulator element q of lane l.
//
// Work decomposition: grid.y walks the tile list (expert, first row) built
// by the router; grid.x walks spans of output columns; each wave owns 16*MB
// rows and NCB 16-column blocks.  Gate/up waves own matching gate and up
// columns, so the epilogue has both halves of h in the same lane.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

__device__ __forceinline__ float clamped_swiglu(float g, float u, float c) {
  const float gc = (g != g) ? g : fminf(fmaxf(g, -c), c);
  const float uc = (u != u) ? u : fminf(fmaxf(u, -c), c);
  return gc / (1.0f + expf(-gc)) * (uc + 1.0f);
}

template <int MB, int NCB, int NW, bool GATEUP>
__global__ __launch_bounds__(NW * 64) void expert_gemm_kernel(GemmParams p) {
  constexpr int HALF = NCB / 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.y;
  if (tile >= *p.n_tiles) return;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int rows = min(16 * MB, p.counts[e] - m0);
  const int row_base = p.offsets[e] + m0;
  const int K = p.K, N = p.N, I = p.I;
  const int nblk = K >> 5;
  const int g = lane >> 4, r = lane & 15;
  const int unit = blockIdx.x * NW + wave;

  // ---- output columns of this wave ---------------------------------------
  int col0;  // first gate column (gate/up) or first output column (down)
  int brow[NCB];
  bool bok[NCB];
  if (GATEUP) {
    col0 = unit * HALF * 16;
#pragma unroll
    for (int j = 0; j < HALF; ++j) {
      bok[j] = bok[HALF + j] = (col0 + 16 * j) < I;
      brow[j] = col0 + 16 * j + r;
      brow[HALF + j] = I + col0 + 16 * j + r;
    }
  } else {
    col0 = unit * NCB * 16;
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      bok[j] = (col0 + 16 * j) < N;
      brow[j] = col0 + 16 * j + r;
    }
  }
  if (!bok[0]) return;

  const uint8_t* bcode[NCB];
  const uint8_t* bscale[NCB];
#pragma unroll
  for (int j = 0; j < NCB; ++j) {
    const size_t rr = (size_t)e * N + (bok[j] ? brow[j] : 0);
    bcode[j] = p.b_codes + rr * (size_t)(K >> 1) + 16 * g;
    bscale[j] = p.b_scales + rr * (size_t)nblk + g;
  }
  const uint8_t* arow[MB];
  bool aok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int m = 16 * mb + r;
    aok[mb] = m < rows;
    size_t ar = 0;
    if (aok[mb]) {
      if (GATEUP) ar = (size_t)(p.expert_rows[(size_t)e * p.T + m0 + m] / p.k);
      else ar = (size_t)(row_base + m);
    }
    arow[mb] = p.a + (ar * nblk + g) * MX6_BLOCK_BYTES;
  }

  v4f acc[MB][NCB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < NCB; ++j) acc[mb][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int nchunk = (nblk + 3) >> 2;
  uint4 A[MB][5], Bc[NCB];
  int Bs[NCB];
  auto load = [&](int c, uint4 (&a)[MB][5], uint4 (&bc)[NCB], int (&bs)[NCB]) {
    const bool inb = (4 * c + g) < nblk;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (aok[mb] && inb) {
        const uint4* src = (const uint4*)(arow[mb] + (size_t)(4 * c) * MX6_BLOCK_BYTES);
#pragma unroll
        for (int q = 0; q < 5; ++q) a[mb][q] = src[q];
      } else {
#pragma unroll
        for (int q = 0; q < 5; ++q) a[mb][q] = make_uint4(0, 0, 0, 0);
        a[mb][4].z = 0x007f7f7fu;
      }
    }
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      if (bok[j] && inb) {
        bc[j] = *(const uint4*)(bcode[j] + (size_t)(4 * c) * 16);
        bs[j] = bscale[j][4 * c];
      } else {
        bc[j] = make_uint4(0, 0, 0, 0);
        bs[j] = 127;
      }
    }
  };
  load(0, A, Bc, Bs);
  for (int c = 0; c < nchunk; ++c) {
    uint4 An[MB][5], Bn[NCB];
    int Bsn[NCB];
    if (c + 1 < nchunk) load(c + 1, An, Bn, Bsn);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint32_t* aw = (const uint32_t*)&A[mb][0];
      const v8i a0 = {(int)aw[0], (int)aw[1], (int)aw[2], (int)aw[3], (int)aw[4], (int)aw[5], 0, 0};
      const v8i a1 = {(int)aw[6], (int)aw[7], (int)aw[8], (int)aw[9], (int)aw[10], (int)aw[11], 0, 0};
      const v8i a2 = {(int)aw[12], (int)aw[13], (int)aw[14], (int)aw[15], (int)aw[16], (int)aw[17], 0, 0};
      const int sw = (int)aw[18];
      const int s0 = sw & 0xff, s1 = (sw >> 8) & 0xff, s2 = (sw >> 16) & 0xff;
#pragma unroll
      for (int j = 0; j < NCB; ++j) {
        const v8i b = {(int)Bc[j].x, (int)Bc[j].y, (int)Bc[j].z, (int)Bc[j].w, 0, 0, 0, 0};
        acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a0, b, acc[mb][j], 2, 4, 0, s0, 0, Bs[j]);
        acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a1, b, acc[mb][j], 2, 4, 0, s1, 0, Bs[j]);
        acc[mb][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a2, b, acc[mb][j], 2, 4, 0, s2, 0, Bs[j]);
      }
    }
    if (c + 1 < nchunk) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q = 0; q < 5; ++q) A[mb][q] = An[mb][q];
#pragma unroll
      for (int j = 0; j < NCB; ++j) { Bc[j] = Bn[j]; Bs[j] = Bsn[j]; }
    }
  }

  if (!GATEUP) {
    // ---- down epilogue: + b2, fp32 rows in permuted order ------------------
#pragma unroll
    for (int j = 0; j < NCB; ++j) {
      if (!bok[j]) continue;
      const int col = col0 + 16 * j + r;
      const float bias = p.bias[(size_t)e * N + col];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 16 * mb + 4 * g + q;
          if (row < rows) p.y[(size_t)(row_base + row) * N + col] = acc[mb][j][q] + bias;
        }
    }
    return;
  }

  // ---- gate/up epilogue: + b13, clamped SwiGLU, MX6x3 split of h ----------
  __shared__ uint8_t s_codes[NW][16][3][32];
  __shared__ uint32_t s_sc[NW][16];
  const int iblocks = I >> 5;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int pp = 0; pp < HALF / 2; ++pp) {
      if (!bok[2 * pp]) continue;
      const int c0 = col0 + 32 * pp + r;
      const float bg0 = p.bias[(size_t)e * N + c0], bg1 = p.bias[(size_t)e * N + c0 + 16];
      const float bu0 = p.bias[(size_t)e * N + I + c0], bu1 = p.bias[(size_t)e * N + I + c0 + 16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float h0 = clamped_swiglu(acc[mb][2 * pp][q] + bg0, acc[mb][HALF + 2 * pp][q] + bu0, p.clamp);
        float h1 = clamped_swiglu(acc[mb][2 * pp + 1][q] + bg1, acc[mb][HALF + 2 * pp + 1][q] + bu1, p.clamp);
        const int row = 4 * g + q;
        uint32_t scw = 0;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          float amax = fmaxf(fabsf(h0), fabsf(h1));
          if (h0 != h0 || h1 != h1) amax = __builtin_inff();
#pragma unroll
          for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
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
          s_codes[wave][row][t][r] = (uint8_t)k0;
          s_codes[wave][row][t][16 + r] = (uint8_t)k1;
        }
        if (r == 0) s_sc[wave][row] = scw;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int blk = (col0 >> 5) + pp;
      if (lane < 48) {
        const int row = lane / 3, t = lane - 3 * (lane / 3);
        if (16 * mb + row < rows) {
          uint8_t cc[32];
#pragma unroll
          for (int i = 0; i < 32; ++i) cc[i] = s_codes[wave][row][t][i];
          uint32_t pk[6];
          pack6x32(cc, pk);
          uint2* dst = (uint2*)(p.hq + ((size_t)(row_base + 16 * mb + row) * iblocks + blk) * MX6_BLOCK_BYTES + 24 * t);
          dst[0] = make_uint2(pk[0], pk[1]);
          dst[1] = make_uint2(pk[2], pk[3]);
          dst[2] = make_uint2(pk[4], pk[5]);
        }
      } else {
        const int row = lane - 48;
        if (16 * mb + row < rows) {
          uint2* dst = (uint2*)(p.hq + ((size_t)(row_base + 16 * mb + row) * iblocks + blk) * MX6_BLOCK_BYTES + 72);
          dst[0] = make_uint2(s_sc[wave][row], 0u);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

// configurations: (MB, NCB, NW)
//   small-M (about 16 rows per expert, decode): one 16-row block per wave,
//     many narrow column spans so that every CU streams weights;
//   large-M (prefill): four 16-row blocks per wave.
int launch_gemm_gateup(const GemmParams& p, int max_tiles, bool small_m, hipStream_t s) {
  if (small_m) {
    constexpr int MB = 1, NCB = 4, NW = 3;
    const int span = NW * (NCB / 2) * 16;
    dim3 grid((p.I + span - 1) / span, max_tiles);
    hipLaunchKernelGGL((expert_gemm_kernel<MB, NCB, NW, true>), grid, dim3(NW * 64), 0, s, p);
  } else {
    constexpr int MB = 4, NCB = 4, NW = 4;
    const int span = NW * (NCB / 2) * 16;
    dim3 grid((p.I + span - 1) / span, max_tiles);
    hipLaunchKernelGGL((expert_gemm_kernel<MB, NCB, NW, true>), grid, dim3(NW * 64), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_gemm_down(const GemmParams& p, int max_tiles, bool small_m, hipStream_t s) {
  if (small_m) {
    constexpr int MB = 1, NCB = 2, NW = 3;
    const int span = NW * NCB * 16;
    dim3 grid((p.N + span - 1) / span, max_tiles);
    hipLaunchKernelGGL((expert_gemm_kernel<MB, NCB, NW, false>), grid, dim3(NW * 64), 0, s, p);
  } else {
    constexpr int MB = 4, NCB = 4, NW = 4;
    const int span = NW * NCB * 16;
    dim3 grid((p.N + span - 1) / span, max_tiles);
    hipLaunchKernelGGL((expert_gemm_kernel<MB, NCB, NW, false>), grid, dim3(NW * 64), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
