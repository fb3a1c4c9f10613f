// Weighted combine of the k expert outputs of every token, and the
// residual + RMSNorm step of the layer stack.
//
// out[t] = sum over slots j (in slot order) of w[t,j] * z[t,j], where z[t,j]
// is the expert output row of pair (t, j) in the expert-grouped buffer
// ("OpenAI 最新开源模型 gpt-oss 架构与训练解析", 模型架构: MoE item, softmax
// weighting of the chosen experts).  RMSNorm divides by the root mean square
// with no bias or shift (same page, RMSNorm 替换 LayerNorm).
//
// The plain combine has one thread per float4 column group of a token.  The
// row kernels of the stack (the combine with the residual add and RMSNorm,
// the residual add + RMSNorm on its own, and RMSNorm) give each row one
// 256-thread workgroup: thread i handles float4 column groups i, i + 256,
// ...; the row's sum of squares is reduced the same way in all three
// (within each wave, then the four waves' sums in wave order), so the stack
// entry point equals its steps bit for bit.
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

constexpr int ROW_THREADS = 256;
constexpr int ROW_KEEP = 4;  // float4 groups per thread kept in registers (rows up to 4096 wide)

// Sum over the row's 256 threads of each thread's partial sum of squares:
// within each wave (butterfly), then the four waves' sums in wave order.
__device__ __forceinline__ float row_sum(float v, float* s_red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  return ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
}

__device__ __forceinline__ float rms_scale(float ss, int d, float eps) { return 1.0f / sqrtf(ss / (float)d + eps); }

__device__ __forceinline__ float sumsq4(float4 v) { return v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w; }

// The RMSNorm pass of one row: no[c] = bf16(x[c] * inv) for this thread's
// groups; the first ROW_KEEP come from registers (xk), later ones are re-read
// from xr, which this same thread wrote or read earlier.
__device__ __forceinline__ void norm_row(const uint16_t* xr, uint16_t* no, const float4 (&xk)[ROW_KEEP], float inv,
                                         int d4) {
  int i = 0;
  for (int c = threadIdx.x; c < d4; c += ROW_THREADS, ++i) {
    float4 x;
    if (i < ROW_KEEP) {
#pragma unroll
      for (int q = 0; q < ROW_KEEP; ++q)
        if (q == i) x = xk[q];
    } else {
      x = unpack_bf16x4(((const uint2*)xr)[c]);
    }
    ((uint2*)no)[c] = pack_bf16x4(make_float4(x.x * inv, x.y * inv, x.z * inv, x.w * inv));
  }
}

__device__ __forceinline__ void keep(float4 (&xk)[ROW_KEEP], int i, float4 v) {
#pragma unroll
  for (int q = 0; q < ROW_KEEP; ++q)
    if (q == i) xk[q] = v;
}

// Stack variant of the combine, one row per workgroup: the combine sum,
// x_out = bf16(x + sum) (the add in fp32) and, unless it is the last layer,
// n_out = bf16(RMSNorm(x_out)).  K: the slots per token (a template
// argument, so that every slot's loads are issued before the first sum).
template <int K>
__global__ __launch_bounds__(ROW_THREADS) void combine_kernel(CombineParams p) {
  __shared__ float s_red[ROW_THREADS / 64];
  const int t = blockIdx.x;
  const int k = K, d = p.d, d4 = d >> 2;
  const float4* rows[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < k; ++j) {
    const int pair = t * k + j;
    const int e = p.topk_id[pair];
    rows[j] = (const float4*)(p.y + (size_t)(p.offsets[e] + p.rel_pos[pair]) * d);
    w[j] = p.topk_w[pair];
  }
  const uint2* xi = (const uint2*)(p.resid_in + (size_t)t * d);
  uint2* xo = (uint2*)(p.resid_out + (size_t)t * d);
  float ss = 0.f;
  float4 xk[ROW_KEEP];
  int i = 0;
  for (int c = threadIdx.x; c < d4; c += ROW_THREADS, ++i) {
    const uint2 xr = xi[c];  // (in flight with the rows' loads)
    float4 v[K];
#pragma unroll
    for (int j = 0; j < k; ++j) v[j] = rows[j][c];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < k; ++j) {
      acc.x = fmaf(w[j], v[j].x, acc.x);
      acc.y = fmaf(w[j], v[j].y, acc.y);
      acc.z = fmaf(w[j], v[j].z, acc.z);
      acc.w = fmaf(w[j], v[j].w, acc.w);
    }
    if (p.out_f32) ((float4*)(p.out_f32 + (size_t)t * d))[c] = acc;
    if (p.out) ((uint2*)(p.out + (size_t)t * d))[c] = pack_bf16x4(acc);
    const float4 x = unpack_bf16x4(xr);
    const uint2 xb = pack_bf16x4(make_float4(x.x + acc.x, x.y + acc.y, x.z + acc.z, x.w + acc.w));
    xo[c] = xb;
    const float4 xn = unpack_bf16x4(xb);
    keep(xk, i, xn);
    ss += sumsq4(xn);
  }
  if (p.norm_out == nullptr) return;
  const float inv = rms_scale(row_sum(ss, s_red), d, p.eps);
  norm_row(p.resid_out + (size_t)t * d, p.norm_out + (size_t)t * d, xk, inv, d4);
}

// The residual add and RMSNorm on their own, one row per workgroup:
// x_out = bf16(x + y), n_out = bf16(RMSNorm(x_out)); y is bf16 or fp32.
template <bool YF32>
__global__ __launch_bounds__(ROW_THREADS) void residual_rmsnorm_kernel(const uint16_t* x, const void* y,
                                                                       uint16_t* x_out, uint16_t* n_out, int T, int d,
                                                                       float eps) {
  __shared__ float s_red[ROW_THREADS / 64];
  const int t = blockIdx.x, d4 = d >> 2;
  const size_t ro = (size_t)t * d;
  const uint2* xi = (const uint2*)(x + ro);
  uint2* xo = (uint2*)(x_out + ro);
  float ss = 0.f;
  float4 xk[ROW_KEEP];
  int i = 0;
  for (int c = threadIdx.x; c < d4; c += ROW_THREADS, ++i) {
    const float4 a = YF32 ? ((const float4*)((const float*)y + ro))[c]
                          : unpack_bf16x4(((const uint2*)((const uint16_t*)y + ro))[c]);
    const float4 xv = unpack_bf16x4(xi[c]);
    const uint2 xb = pack_bf16x4(make_float4(xv.x + a.x, xv.y + a.y, xv.z + a.z, xv.w + a.w));
    xo[c] = xb;
    const float4 xn = unpack_bf16x4(xb);
    keep(xk, i, xn);
    ss += sumsq4(xn);
  }
  if (n_out == nullptr) return;
  const float inv = rms_scale(row_sum(ss, s_red), d, eps);
  norm_row(x_out + ro, n_out + ro, xk, inv, d4);
}

// Plain combine: one thread per float4 column group of one token, so that a
// small batch still spreads over many workgroups.
// K: the slots per token (a template argument, so that every slot's loads
// are issued before the first sum).
template <int K>
__global__ __launch_bounds__(256) void combine_cols_kernel(CombineParams p) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int k = K, d = p.d;
  if (c >= (d >> 2)) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
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

// RMSNorm of one row per workgroup (out may equal x: every thread reads its
// groups before the barrier inside row_sum and rewrites only its own).
__global__ __launch_bounds__(ROW_THREADS) void rmsnorm_kernel(const uint16_t* x, uint16_t* out, int T, int d,
                                                             float eps) {
  __shared__ float s_red[ROW_THREADS / 64];
  const int t = blockIdx.x, d4 = d >> 2;
  const uint2* xr = (const uint2*)(x + (size_t)t * d);
  float ss = 0.f;
  float4 xk[ROW_KEEP];
  int i = 0;
  for (int c = threadIdx.x; c < d4; c += ROW_THREADS, ++i) {
    const float4 v = unpack_bf16x4(xr[c]);
    keep(xk, i, v);
    ss += sumsq4(v);
  }
  const float inv = rms_scale(row_sum(ss, s_red), d, eps);
  norm_row(x + (size_t)t * d, out + (size_t)t * d, xk, inv, d4);
}

__global__ void zero_ints_kernel(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

int launch_combine(const CombineParams& p, hipStream_t s) {
  const dim3 gc((p.d / 4 + 255) / 256, p.T), gr(p.T);
#define MOE_COMB(K)                                                                    \
  if (p.resid_out == nullptr)                                                          \
    hipLaunchKernelGGL(combine_cols_kernel<K>, gc, dim3(256), 0, s, p);                \
  else                                                                                 \
    hipLaunchKernelGGL(combine_kernel<K>, gr, dim3(ROW_THREADS), 0, s, p);
  switch (p.k) {
    case 1: MOE_COMB(1) break;
    case 2: MOE_COMB(2) break;
    case 3: MOE_COMB(3) break;
    case 4: MOE_COMB(4) break;
    case 5: MOE_COMB(5) break;
    case 6: MOE_COMB(6) break;
    case 7: MOE_COMB(7) break;
    case 8: MOE_COMB(8) break;
    default: return -1;
  }
#undef MOE_COMB
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_rmsnorm(const uint16_t* x, uint16_t* out, int T, int d, float eps, hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(T), dim3(ROW_THREADS), 0, s, x, out, T, d, eps);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_residual_rmsnorm(const uint16_t* x, const void* y, bool y_f32, uint16_t* x_out, uint16_t* n_out, int T,
                            int d, float eps, hipStream_t s) {
  const dim3 g(T), b(ROW_THREADS);
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
