// Bit-exact code checks: write the codes the fused kernels see, through the
// very same register-level extraction routines (q3_block_pairs,
// q4_word_pairs), as int8 [K, N].  A thread takes 4 columns (one 128-bit
// word row) of one 32-row block (3-bit) or one 8-row word (4-bit).
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 255) | ((uint32_t)(b & 255) << 8) | ((uint32_t)(c & 255) << 16) |
         ((uint32_t)(d & 255) << 24);
}

__global__ __launch_bounds__(kThreads) void unpack_q3_kernel(const uint32_t* __restrict__ qw,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N) {
  const int n4 = N / 4;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)(K / 32) * n4) return;
  const int blk = (int)(idx / n4), col0 = (int)(idx % n4) * 4;
  u32x4 w[3];
#pragma unroll
  for (int j = 0; j < 3; ++j)
    w[j] = *reinterpret_cast<const u32x4*>(qw + (size_t)(3 * blk + j) * N + col0);
  h2 pr[4][16];
#pragma unroll
  for (int c = 0; c < 4; ++c) q3_block_pairs(w[0][c], w[1][c], w[2][c], pr[c]);
#pragma unroll
  for (int P = 0; P < 16; ++P) {
    const int ra = 32 * blk + q3_pair(P).a, rb = 32 * blk + q3_pair(P).b;
    *reinterpret_cast<uint32_t*>(codes + (size_t)ra * N + col0) =
        pack4_i8((int)pr[0][P].x, (int)pr[1][P].x, (int)pr[2][P].x, (int)pr[3][P].x);
    *reinterpret_cast<uint32_t*>(codes + (size_t)rb * N + col0) =
        pack4_i8((int)pr[0][P].y, (int)pr[1][P].y, (int)pr[2][P].y, (int)pr[3][P].y);
  }
}

__global__ __launch_bounds__(kThreads) void unpack_q4_kernel(const uint32_t* __restrict__ qw,
                                                             const int* __restrict__ perm,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N) {
  const int n4 = N / 4;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)(K / 8) * n4) return;
  const int r = (int)(idx / n4), col0 = (int)(idx % n4) * 4;
  const u32x4 w = *reinterpret_cast<const u32x4*>(qw + (size_t)r * N + col0);
  h2 pr[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c) q4_word_pairs(w[c], pr[c]);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ia = 8 * r + j, ib = ia + 4;
    const int da = perm ? perm[ia] : ia, db = perm ? perm[ib] : ib;
    *reinterpret_cast<uint32_t*>(codes + (size_t)da * N + col0) =
        pack4_i8((int)pr[0][j].x, (int)pr[1][j].x, (int)pr[2][j].x, (int)pr[3][j].x);
    *reinterpret_cast<uint32_t*>(codes + (size_t)db * N + col0) =
        pack4_i8((int)pr[0][j].y, (int)pr[1][j].y, (int)pr[2][j].y, (int)pr[3][j].y);
  }
}

hipError_t launch_unpack_q3(const int32_t* qw, int8_t* codes, int K, int N, hipStream_t s) {
  const size_t total = (size_t)(K / 32) * (N / 4);
  hipLaunchKernelGGL(unpack_q3_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(qw), codes, K, N);
  return hipGetLastError();
}

hipError_t launch_unpack_q4(const int32_t* qw, const int32_t* perm, int8_t* codes, int K, int N,
                            hipStream_t s) {
  const size_t total = (size_t)(K / 8) * (N / 4);
  hipLaunchKernelGGL(unpack_q4_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(qw), perm, codes, K,
                     N);
  return hipGetLastError();
}

}  // namespace wq
