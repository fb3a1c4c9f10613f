// Repacks MXFP4 weight stacks (the stored format, [E, N, K/2] E2M1 codes and
// [E, N, K/32] E8M0 scale bytes, row-major; "OpenAI 最新开源模型 gpt-oss 架构与
// 训练解析", 权重量化 item) into the layout the wide prefill GEMM streams:
//
//   codes   the K dimension goes in chunks of four 32-element blocks (64
//           bytes of a row); for each pair of consecutive weight rows
//           (2p, 2p + 1) and chunk c, row 2p's chunk segment is followed by
//           row 2p + 1's, so one 128-byte line holds what one chunk of the
//           GEMM reads from two rows.  A pair takes K bytes; a short last
//           chunk (K/32 not a multiple of 4) keeps its 2 x 16 (K/32 - 4c)
//           bytes in the same order.
//   scales  chunk-major: for each chunk c, 4 bytes per weight row (the
//           scales of blocks 4c .. 4c + 3, rows consecutive), so a chunk's
//           scales of 64 consecutive rows are 256 contiguous bytes; blocks
//           past K/32 hold 127 (scale 1), never used with a non-zero
//           activation.
//
// Nothing is converted: every byte keeps its value.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// one thread per 16-byte block of the input codes
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* codes, uint8_t* out, int N, int K,
                                                         long long blocks) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= blocks) return;
  const int nblk = K >> 5;
  const long long row = i / nblk;          // e * N + n
  const int b = (int)(i - row * nblk);
  const int n = (int)(row % N);
  const long long e = row / N;
  const int c = b >> 2;
  const int w = 16 * min(4, nblk - 4 * c);
  const size_t dst = (size_t)e * N * (K >> 1) + (size_t)(n >> 1) * K + 128 * (size_t)c + (size_t)(n & 1) * w +
                     16 * (size_t)(b & 3);
  *(uint4*)(out + dst) = *(const uint4*)(codes + (size_t)row * (K >> 1) + 16 * (size_t)b);
}

// one thread per output dword: chunk c of weight row n of expert e
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint8_t* scales, uint8_t* out, int N, int nblk,
                                                          long long dwords) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= dwords) return;
  const int nchk = (nblk + 3) >> 2;
  const int n = (int)(i % N);
  const long long ec = i / N;              // e * nchk + c
  const int c = (int)(ec % nchk);
  const long long e = ec / nchk;
  const uint8_t* src = scales + ((size_t)e * N + n) * nblk;
  uint32_t v = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = 4 * c + q;
    v |= (uint32_t)(b < nblk ? src[b] : (uint8_t)127) << (8 * q);
  }
  ((uint32_t*)out)[i] = v;
}

int launch_pack_weights(const uint8_t* codes, const uint8_t* scales, int E, int N, int K, uint8_t* codes_out,
                        uint8_t* scales_out, hipStream_t s) {
  const int nblk = K >> 5, nchk = (nblk + 3) >> 2;
  const long long blocks = (long long)E * N * nblk;
  const long long dwords = (long long)E * nchk * N;
  hipLaunchKernelGGL(pack_codes_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s, codes, codes_out,
                     N, K, blocks);
  hipLaunchKernelGGL(pack_scales_kernel, dim3((unsigned)((dwords + 255) / 256)), dim3(256), 0, s, scales,
                     scales_out, N, nblk, dwords);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace moe
