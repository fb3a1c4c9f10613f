// Weighted combine of the k expert outputs of every token, and the
// residual + RMSNorm step of the layer stack.
//
// out[t] = sum over slots j (in slot order) of w[t,j] * z[t,j], where z[t,j]
// is the expert output row of pair (t, j) in the expert-grouped buffer
// ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", 模型架构: MoE item, softmax
// weighting of the chosen experts).  RMSNorm divides by the root mean square
// with no bias or shift (same page, RMSNorm 替换 LayerNorm).
//
// One wave per token; every lane handles float4 column groups, so each
// expert row is read with fully coalesced 16-byte loads.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

__device__ __forceinline__ uint2 pack_bf16x4(float4 v) {
  return make_uint2((uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                    (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16));
}
__device__ __forceinline__ float4 unpack_bf16x4(uint2 u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Residual step of the pre-norm stack for one float4 column group c of a
// row: xo[c] = bf16(xi[c] + add) with the add in fp32; returns the sum of
// squares of the rounded values (the RMSNorm statistic).
__device__ __forceinline__ float residual_add4(const uint16_t* xi, uint16_t* xo, int c, float4 add) {
  const float4 x = unpack_bf16x4(((const uint2*)xi)[c]);
  const uint2 xb = pack_bf16x4(make_float4(x.x + add.x, x.y + add.y, x.z + add.z, x.w + add.w));
  ((uint2*)xo)[c] = xb;
  const float4 xn = unpack_bf16x4(xb);
  return xn.x * xn.x + xn.y * xn.y + xn.z * xn.z + xn.w * xn.w;
}

// Second pass of the RMSNorm of one row held by one wave: no = bf16(xr *
// 1/sqrt(ss/d + eps)), ss the wave's summed squares (reduced here).
__device__ __forceinline__ void rmsnorm_row(const uint16_t* xr, uint16_t* no, float ss, int d, float eps, int lane) {
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  for (int c = lane; c < (d >> 2); c += 64) {
    const float4 x = unpack_bf16x4(((const uint2*)xr)[c]);
    ((uint2*)no)[c] = pack_bf16x4(make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv));
  }
}

__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int k = p.k, d = p.d, d4 = d >> 2;
  const float4* rows[8];
  float w[8];
  for (int j = 0; j < k; ++j) {
    const int pair = t * k + j;
    const int e = p.topk_id[pair];
    rows[j] = (const float4*)(p.y + (size_t)(p.offsets[e] + p.rel_pos[pair]) * d);
    w[j] = p.topk_w[pair];
  }
  const bool stack = p.resid_out != nullptr;
  float ss = 0.f;
  for (int c = lane; c < d4; c += 64) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float4 v = rows[j][c];
      acc.x = fmaf(w[j], v.x, acc.x);
      acc.y = fmaf(w[j], v.y, acc.y);
      acc.z = fmaf(w[j], v.z, acc.z);
      acc.w = fmaf(w[j], v.w, acc.w);
    }
    if (p.out_f32) ((float4*)(p.out_f32 + (size_t)t * d))[c] = acc;
    if (p.out) ((uint2*)(p.out + (size_t)t * d))[c] = pack_bf16x4(acc);
    if (stack) ss += residual_add4(p.resid_in + (size_t)t * d, p.resid_out + (size_t)t * d, c, acc);
  }
  if (!stack || p.norm_out == nullptr) return;
  rmsnorm_row(p.resid_out + (size_t)t * d, p.norm_out + (size_t)t * d, ss, d, p.eps, lane);
}

// The residual add and RMSNorm on their own (one wave per row): x_out =
// bf16(x + y), n_out = bf16(RMSNorm(x_out)); y is bf16 or fp32.
template <bool YF32>
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(const uint16_t* x, const void* y, uint16_t* x_out,
                                                               uint16_t* n_out, int T, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t ro = (size_t)t * d;
  float ss = 0.f;
  for (int c = lane; c < (d >> 2); c += 64) {
    const float4 a = YF32 ? ((const float4*)((const float*)y + ro))[c]
                          : unpack_bf16x4(((const uint2*)((const uint16_t*)y + ro))[c]);
    ss += residual_add4(x + ro, x_out + ro, c, a);
  }
  if (n_out != nullptr) rmsnorm_row(x_out + ro, n_out + ro, ss, d, eps, lane);
}

// Plain combine: one thread per float4 column group of one token, so that a
// small batch still spreads over many workgroups.
__global__ __launch_bounds__(256) void combine_cols_kernel(CombineParams p) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int k = p.k, d = p.d;
  if (c >= (d >> 2)) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int pair = t * k + j;
    const float w = p.topk_w[pair];
    const float4 v = ((const float4*)(p.y + (size_t)(p.offsets[p.topk_id[pair]] + p.rel_pos[pair]) * d))[c];
    acc.x = fmaf(w, v.x, acc.x);
    acc.y = fmaf(w, v.y, acc.y);
    acc.z = fmaf(w, v.z, acc.z);
    acc.w = fmaf(w, v.w, acc.w);
  }
  if (p.out_f32) ((float4*)(p.out_f32 + (size_t)t * d))[c] = acc;
  if (p.out) ((uint2*)(p.out + (size_t)t * d))[c] = pack_bf16x4(acc);
}

__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* x, uint16_t* out, int T, int d, float eps) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int d4 = d >> 2;
  const uint2* xr = (const uint2*)(x + (size_t)t * d);
  float ss = 0.f;
  for (int c = lane; c < d4; c += 64) {
    const float4 v = unpack_bf16x4(xr[c]);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  uint2* orow = (uint2*)(out + (size_t)t * d);
  for (int c = lane; c < d4; c += 64) {
    const float4 v = unpack_bf16x4(xr[c]);
    orow[c] = pack_bf16x4(make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv));
  }
}

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

int launch_combine(const CombineParams& p, hipStream_t s) {
  if (p.resid_out == nullptr) {
    hipLaunchKernelGGL(combine_cols_kernel, dim3((p.d / 4 + 255) / 256, p.T), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(combine_kernel, dim3((p.T + 3) / 4), dim3(256), 0, s, p);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_rmsnorm(const uint16_t* x, uint16_t* out, int T, int d, float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((T + 3) / 4), dim3(256), 0, s, x, out, T, d, eps);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_residual_rmsnorm(const uint16_t* x, const void* y, bool y_f32, uint16_t* x_out, uint16_t* n_out, int T,
                            int d, float eps, hipStream_t s) {
  const dim3 g((T + 3) / 4), b(256);
  if (y_f32)
    hipLaunchKernelGGL(residual_rmsnorm_kernel<true>, g, b, 0, s, x, y, x_out, n_out, T, d, eps);
  else
    hipLaunchKernelGGL(residual_rmsnorm_kernel<false>, g, b, 0, s, x, y, x_out, n_out, T, d, eps);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_zero_ints(int* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_ints_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
