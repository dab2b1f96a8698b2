// 4-bit symmetric group-wise weight-only GEMM (small M), with act-order.
//
//   Y[m, n] = sum_g scale[g, n] * sum_{rows i of group g} X[m, perm[i]] * q'[i, n]
//
// Codes are 8 per int32 along K, stored as q + 8 ("Quantization CUDA",
// tom-jerr.github.io, sections "Int4 Weight Only Quantization" and "Weight
// Store"; "量化粒度": group-wise scales, groups of 128 along K).  With
// act-order ("GPTQ算法解析", intelliparadigm.com, section 4.1: act_order) a
// row's group is g_idx[k], which is not monotone in k.  The weight is
// reordered once, offline, so that the rows of each group are contiguous
// (wq_q4_prepack, the same idea as the offline re-layout of "Marlin 格式" on
// the "Quantization CUDA" page); the kernel then gathers the activations
// through perm while staging them, and every span of rows it reads belongs to
// a single group whose scale is applied once.
//
// Geometry.  A workgroup (4 wave64s) owns a 256-column tile (4 columns per
// lane) and 4*WPW word rows (32*WPW rows of K); wave w takes WPW word rows,
// which lie in one group (8*WPW divides G).  Each code pair is reused for all
// M rows of X.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

template <int MT, int WPW>
__global__ __launch_bounds__(kThreads) void q4_group_kernel(
    const _Float16* __restrict__ X, const uint32_t* __restrict__ qw,
    const _Float16* __restrict__ scales, const int* __restrict__ perm, _Float16* __restrict__ Y,
    float* __restrict__ part, unsigned* __restrict__ counters, int M, int K, int N, int G, int S) {
  constexpr int RPG = 4 * WPW;  // word rows per workgroup
  __shared__ h2 xs[MT][RPG][4];
  __shared__ float red[4][MT][kTileN + 4];
  __shared__ int last_flag;

  const int nr = K / 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ct = blockIdx.x / S, s = blockIdx.x % S;
  const int r0 = s * RPG;
  const int col0 = ct * kTileN + lane * 4;
  const bool col_ok = col0 < N;
  const int rw0 = r0 + wave * WPW;  // this wave's first word row

  // 1. Stream this wave's word rows (rows past the end read as zero).
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(qw, nr * N * 4);
  u32x4 w[WPW];
#pragma unroll
  for (int i = 0; i < WPW; ++i)
    w[i] = buffer_stream(wr, col_ok ? ((rw0 + i) * N + col0) * 4 : kOutOfRange);

  // 2. Stage X[m, perm[i]] as the pairs (rows 8r+j, 8r+j+4) the codes come in.
  for (int idx = tid; idx < MT * RPG * 4; idx += kThreads) {
    const int m = idx / (RPG * 4), rem = idx % (RPG * 4);
    const int rw = rem >> 2, j = rem & 3;
    const int ia = 8 * (r0 + rw) + j, ib = ia + 4;
    _Float16 a = 0, b = 0;
    if (m < M && ia < K) {
      const int ka = perm ? perm[ia] : ia, kb = perm ? perm[ib] : ib;
      a = X[(size_t)m * K + ka];
      b = X[(size_t)m * K + kb];
    }
    xs[m][rw][j] = (h2){a, b};
  }
  __syncthreads();

  // 3. Exact codes, fp32 accumulation.
  float acc[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m][c] = 0.0f;
#pragma unroll
  for (int i = 0; i < WPW; ++i) {
    h2 xv[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) xv[m][j] = xs[m][wave * WPW + i][j];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      h2 pr[4];
      q4_word_pairs(w[i][c], pr);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][c] = dot2(pr[j], xv[m][j], acc[m][c]);
    }
  }

  // 4. The span is one group: scale once.
  if (col_ok && 8 * rw0 < K) {
    const uint2 sraw = *reinterpret_cast<const uint2*>(scales + (size_t)((8 * rw0) / G) * N + col0);
    const h2 s01 = as_h2(sraw.x), s23 = as_h2(sraw.y);
    const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[m][c] *= sc[c];
  }

  // 5. Across waves; thread t owns column t of the tile.
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) red[wave][m][lane * 4 + c] = acc[m][c];
  __syncthreads();
  const int n = ct * kTileN + tid;
  float sum[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    sum[m] = (red[0][m][tid] + red[1][m][tid]) + (red[2][m][tid] + red[3][m][tid]);

  if (S == 1) {
    if (n < N)
#pragma unroll
      for (int m = 0; m < MT; ++m)
        if (m < M) Y[(size_t)m * N + n] = (_Float16)sum[m];
    return;
  }
  if (n < N)
#pragma unroll
    for (int m = 0; m < MT; ++m)
      if (m < M) part[((size_t)s * MT + m) * N + n] = sum[m];
  if (splitk_arrive(&counters[ct], S, &last_flag)) {
    if (n < N) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m >= M) continue;
        float t = 0.0f;
        for (int j = 0; j < S; ++j) t += part[((size_t)j * MT + m) * N + n];
        Y[(size_t)m * N + n] = (_Float16)t;
      }
    }
    splitk_reset(&counters[ct]);
  }
}

// Word rows per wave: one whole group when it is at most 128 rows (16 loads
// of 128 bits in flight per lane), else 16.
SplitPlan plan_q4(int M, int K, int N, int G) {
  SplitPlan p;
  p.mt = M == 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8));
  p.n_tiles = (N + kTileN - 1) / kTileN;
  int wpw = G / 8 >= 16 ? 16 : G / 8;  // G % 32 == 0, so wpw is 4, 8 or 16
  const int ov = env_unit_override();
  if ((ov == 4 || ov == 8 || ov == 16) && (G / 8) % ov == 0) wpw = ov;
  p.unit = wpw;
  const int nr = K / 8;
  p.splits = (nr + 4 * wpw - 1) / (4 * wpw);
  return p;
}

template <int MT, int WPW>
static hipError_t launch_q4_t(const void* X, const int32_t* qw, const void* scales,
                              const int32_t* perm, void* Y, int M, int K, int N, int G,
                              const SplitPlan& p, void* ws, hipStream_t s) {
  unsigned* counters = reinterpret_cast<unsigned*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ws_counter_bytes(p.n_tiles));
  hipLaunchKernelGGL((q4_group_kernel<MT, WPW>), dim3(p.n_tiles * p.splits), dim3(kThreads), 0, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint32_t*>(qw),
                     reinterpret_cast<const _Float16*>(scales), perm,
                     reinterpret_cast<_Float16*>(Y), part, counters, M, K, N, G, p.splits);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_q4_mt(const void* X, const int32_t* qw, const void* scales,
                               const int32_t* perm, void* Y, int M, int K, int N, int G,
                               const SplitPlan& p, void* ws, hipStream_t s) {
  switch (p.unit) {
    case 4: return launch_q4_t<MT, 4>(X, qw, scales, perm, Y, M, K, N, G, p, ws, s);
    case 8: return launch_q4_t<MT, 8>(X, qw, scales, perm, Y, M, K, N, G, p, ws, s);
    default: return launch_q4_t<MT, 16>(X, qw, scales, perm, Y, M, K, N, G, p, ws, s);
  }
}

hipError_t launch_q4_group(const void* X, const int32_t* qw, const void* scales,
                           const int32_t* perm, void* Y, int M, int K, int N, int G,
                           const SplitPlan& p, void* ws, hipStream_t s) {
  for (int m0 = 0; m0 < M; m0 += p.mt) {
    const int mc = (M - m0) < p.mt ? (M - m0) : p.mt;
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)m0 * K * 2;
    void* Yc = reinterpret_cast<char*>(Y) + (size_t)m0 * N * 2;
    hipError_t e;
    switch (p.mt) {
      case 1: e = launch_q4_mt<1>(Xc, qw, scales, perm, Yc, mc, K, N, G, p, ws, s); break;
      case 2: e = launch_q4_mt<2>(Xc, qw, scales, perm, Yc, mc, K, N, G, p, ws, s); break;
      case 4: e = launch_q4_mt<4>(Xc, qw, scales, perm, Yc, mc, K, N, G, p, ws, s); break;
      default: e = launch_q4_mt<8>(Xc, qw, scales, perm, Yc, mc, K, N, G, p, ws, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Offline row reorder: out row i = original row perm[i] (one thread per word).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q4_prepack_kernel(const uint32_t* __restrict__ qw,
                                                              const int* __restrict__ perm,
                                                              uint32_t* __restrict__ out, int K,
                                                              int N) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)(K / 8) * N;
  if (idx >= total) return;
  const int r = (int)(idx / N), n = (int)(idx % N);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int src = perm[8 * r + j];
    const uint32_t sw = qw[(size_t)(src >> 3) * N + n];
    word |= ((sw >> (4 * (src & 7))) & 15u) << (4 * j);
  }
  out[idx] = word;
}

hipError_t launch_q4_prepack(const int32_t* qw, const int32_t* perm, int32_t* out, int K, int N,
                             hipStream_t s) {
  const size_t total = (size_t)(K / 8) * N;
  const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(q4_prepack_kernel, dim3(blocks), dim3(kThreads), 0, s,
                     reinterpret_cast<const uint32_t*>(qw), perm, reinterpret_cast<uint32_t*>(out),
                     K, N);
  return hipGetLastError();
}

}  // namespace wq
