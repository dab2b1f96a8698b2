// Group-wise symmetric int8 weight-only GEMV / small-batch GEMM.
//
//   Y[m, n] = sum_g scale[g, n] * sum_{k in group g} X[m, k] * q[k, n]
//
// i.e. Y = X.(Wint*Sw) rearranged as (X.Wint)*Sw per group ("Quantization
// CUDA", tom-jerr.github.io, section "Int8 Weight Only Quantization"), with
// the int8 weight dequantised in registers as it is loaded and never stored
// as floating point ("融合反量化与GEMM：LLM推理的CUDA内核优化实践",
// zingnex.cn, sections "核心优化思路" and "技术实现细节": one fp32 scale per 128
// rows of K per column).
//
// Geometry.  A workgroup (4 wave64s) owns a 256-column tile and TK = 16*R
// rows of K.  Lane (cc, rr) of wave w takes 16 columns (one 128-bit load per
// row) and a contiguous span of R rows: slot = 4w + rr.  R divides the group
// size, so each span lies inside one group and is scaled once.  Every lane
// issues all R of its loads before it converts anything, so the whole tile is
// in flight at once.  Spans are reduced across the 4 lanes of a wave that
// share columns (shuffles) and across the 4 waves (LDS), then across the S
// workgroups of a column tile through the workspace (split-K, fixed order).
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

template <int MT, int R>
__global__ __launch_bounds__(kThreads) void q8_group_kernel(
    const _Float16* __restrict__ X, const int8_t* __restrict__ Wq,
    const float* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ part,
    unsigned* __restrict__ counters, int M, int K, int N, int G, int S) {
  constexpr int TK = 16 * R;
  constexpr int NP = TK / 2;  // row pairs per workgroup
  __shared__ h2 xs[MT][NP];
  __shared__ float red[4][MT][kTileN + 4];
  __shared__ int last_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ct = blockIdx.x / S, s = blockIdx.x % S;
  const int kb = s * TK;
  const int cc = lane & 15, rr = lane >> 4;
  const int slot = wave * 4 + rr;
  const int k0 = kb + slot * R;
  const int col0 = ct * kTileN + cc * 16;
  const bool col_ok = col0 < N;

  // 1. Stream this lane's weight span: R rows x 16 columns.  Rows past K
  //    and columns past N fall outside the buffer range and read as zero.
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wq, K * N);
  const int off0 = col_ok ? k0 * N + col0 : kOutOfRange;
  u32x4 w[R];
#pragma unroll
  for (int i = 0; i < R; ++i) w[i] = buffer_stream(wr, col_ok ? off0 + i * N : kOutOfRange);

  // 2. Stage the activations of this K range as fp16 pairs (rows 2p, 2p+1).
  for (int idx = tid; idx < MT * NP; idx += kThreads) {
    const int m = idx / NP, p = idx % NP;
    const int k = kb + 2 * p;
    uint32_t v = 0;
    if (m < M && k < K) v = *reinterpret_cast<const uint32_t*>(X + (size_t)m * K + k);
    xs[m][p] = as_h2(v);
  }
  __syncthreads();

  // 3. Dequantise in registers and accumulate in fp32.
  float acc[MT][16];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[m][c] = 0.0f;

  const int pbase = slot * (R / 2);
#pragma unroll
  for (int p = 0; p < R / 2; ++p) {
    h2 xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xv[m] = xs[m][pbase + p];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      h2 q[4];
      q8_rowpair_pairs(w[2 * p][d], w[2 * p + 1][d], q);
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m][4 * d + c] = dot2(q[c], xv[m], acc[m][4 * d + c]);
    }
  }

  // 4. One scale per (group, column) for the whole span.
  if (col_ok && k0 < K) {
    const float* sp = scales + (size_t)(k0 / G) * N + col0;
    f32x4 sc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) sc[d] = *reinterpret_cast<const f32x4*>(sp + 4 * d);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[m][c] *= sc[c >> 2][c & 3];
  }

  // 5. Reduce the 4 spans of a wave that share columns (lanes 16 apart).
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      float v = acc[m][c];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      acc[m][c] = v;
    }
  if (rr == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int c = 0; c < 16; ++c) red[wave][m][cc * 16 + c] = acc[m][c];
  }
  __syncthreads();

  // 6. Across the 4 waves; thread t now owns column t of the tile.
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

  // 7. Split-K: publish, and let the last workgroup of the tile finish.
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

// Rows per lane span: as many as the register budget allows (all loads of a
// lane are in flight together), fewer when that leaves too few workgroups.
SplitPlan plan_q8(int M, int K, int N, int G) {
  SplitPlan p;
  p.mt = M == 1 ? 1 : (M == 2 ? 2 : (M <= 4 ? 4 : 8));
  p.n_tiles = (N + kTileN - 1) / kTileN;
  int R = p.mt >= 8 ? 8 : 16;
  const int ov = env_unit_override();
  if (ov == 8 || ov == 16 || (ov == 32 && p.mt <= 2)) R = ov;
  while (R > 8 && G % R) R /= 2;
  if (G % R) R = 8;  // G % 32 == 0 is required by the ABI, so 8 always divides G
  p.unit = R;
  const int TK = 16 * R;
  p.splits = (K + TK - 1) / TK;
  return p;
}

template <int MT, int R>
static hipError_t launch_one(const void* X, const int8_t* Wq, const float* scales, void* Y, int M,
                             int K, int N, int G, const SplitPlan& p, void* ws, hipStream_t s) {
  unsigned* counters = reinterpret_cast<unsigned*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ws_counter_bytes(p.n_tiles));
  hipLaunchKernelGGL((q8_group_kernel<MT, R>), dim3(p.n_tiles * p.splits), dim3(kThreads), 0, s,
                     reinterpret_cast<const _Float16*>(X), Wq, scales,
                     reinterpret_cast<_Float16*>(Y), part, counters, M, K, N, G, p.splits);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_mt(const void* X, const int8_t* Wq, const float* scales, void* Y, int M,
                            int K, int N, int G, const SplitPlan& p, void* ws, hipStream_t s) {
  switch (p.unit) {
    case 8: return launch_one<MT, 8>(X, Wq, scales, Y, M, K, N, G, p, ws, s);
    case 16: return launch_one<MT, 16>(X, Wq, scales, Y, M, K, N, G, p, ws, s);
    default: return launch_one<MT, (MT <= 2 ? 32 : 16)>(X, Wq, scales, Y, M, K, N, G, p, ws, s);
  }
}

hipError_t launch_q8_group(const void* X, const int8_t* Wq, const float* scales, void* Y, int M,
                           int K, int N, int G, const SplitPlan& p, void* ws, hipStream_t s) {
  // Rows of X beyond the per-launch tile height run as further launches.
  for (int m0 = 0; m0 < M; m0 += p.mt) {
    const int mc = (M - m0) < p.mt ? (M - m0) : p.mt;
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)m0 * K * 2;
    void* Yc = reinterpret_cast<char*>(Y) + (size_t)m0 * N * 2;
    hipError_t e;
    switch (p.mt) {
      case 1: e = launch_mt<1>(Xc, Wq, scales, Yc, mc, K, N, G, p, ws, s); break;
      case 2: e = launch_mt<2>(Xc, Wq, scales, Yc, mc, K, N, G, p, ws, s); break;
      case 4: e = launch_mt<4>(Xc, Wq, scales, Yc, mc, K, N, G, p, ws, s); break;
      default: e = launch_mt<8>(Xc, Wq, scales, Yc, mc, K, N, G, p, ws, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
