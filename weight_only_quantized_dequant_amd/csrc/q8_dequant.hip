// The separated (unfused) form of the int8 weight-only product, first half:
// a dequantisation kernel that materialises the whole floating-point weight
//
//   W[k, n] = scale[k / G, n] * q[k, n]      (one fp32 multiply; fp16 output:
//                                             that fp32 product rounded once
//                                             more, to nearest even)
//
// from the stored int8 codes [K, N] and fp32 scales [K/G, N] ("融合反量化与
// GEMM：LLM推理的CUDA内核优化实践", zingnex.cn: section "CUDA内核架构", the
// standalone INT8 -> FP32 dequantisation kernel of the separated pipeline,
// and section "性能对比数据", its "CUDA分离" row).  A general GEMM then reads
// W; the fused products never write it.  Pure streaming: each thread reads
// 16 codes (16 bytes) and their 16 scales, and writes 16 weights.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

constexpr int kDqThreads = 256;

template <bool F16>
__global__ __launch_bounds__(kDqThreads) void q8_dequant_kernel(const int8_t* __restrict__ q,
                                                               const float* __restrict__ scales,
                                                               void* __restrict__ W, int K, int N,
                                                               int G) {
  const size_t t = (size_t)blockIdx.x * kDqThreads + threadIdx.x;
  const int per_row = N / 16;
  if (t >= (size_t)K * per_row) return;
  const int k = (int)(t / per_row), n0 = (int)(t % per_row) * 16;
  const u32x4 codes = *reinterpret_cast<const u32x4*>(q + (size_t)k * N + n0);
  const f32x4* sp = reinterpret_cast<const f32x4*>(scales + (size_t)(k / G) * N + n0);
  float w[16];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const f32x4 sv = sp[v];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int c = (int)(int8_t)((codes[v] >> (8 * e)) & 0xFFu);
      w[4 * v + e] = sv[e] * (float)c;
    }
  }
  if constexpr (F16) {
    u32x4* out = reinterpret_cast<u32x4*>(reinterpret_cast<_Float16*>(W) + (size_t)k * N + n0);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      u32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = as_u32(h2{(_Float16)w[8 * v + 2 * e], (_Float16)w[8 * v + 2 * e + 1]});
      out[v] = o;
    }
  } else {
    f32x4* out = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(W) + (size_t)k * N + n0);
#pragma unroll
    for (int v = 0; v < 4; ++v) out[v] = f32x4{w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]};
  }
}

hipError_t launch_q8_dequant(const int8_t* q, const float* scales, void* W, int K, int N, int G,
                             bool f16, hipStream_t s) {
  const size_t threads = (size_t)K * (N / 16);
  const dim3 grid((unsigned)((threads + kDqThreads - 1) / kDqThreads));
  if (f16)
    hipLaunchKernelGGL(q8_dequant_kernel<true>, grid, dim3(kDqThreads), 0, s, q, scales, W, K, N, G);
  else
    hipLaunchKernelGGL(q8_dequant_kernel<false>, grid, dim3(kDqThreads), 0, s, q, scales, W, K, N, G);
  return hipGetLastError();
}

}  // namespace wq
