// 3-bit GPTQ-style matvec with one scale and one zero per output column.
//
//   y[n] = sum_k x[k] * (scale[n] * q[k, n] - zero[n])
//        = scale[n] * sum_k x[k] * q[k, n]  -  zero[n] * sum_k x[k]
//
// The dequantised weight scale*q - zero is the form of "GPTQ CUDA kernel
// walkthrough" (yelogs.com), section "CUDA核函數設計與實現" (codes shifted and
// masked out of int32 words, one scale and zero per column, the vector cached
// on chip).  Here scale and zero leave the K loop entirely: the loop only
// forms sum_k x[k]*q[k, n] from exact codes, and sum_k x[k] is formed once per
// workgroup.  The same page's "faster" variant packs fp16 activations in
// pairs; the fp16 path here does the same with v_dot2_f32_f16, which
// accumulates in fp32.
//
// Geometry.  A workgroup (4 wave64s) owns a 256-column tile (4 columns per
// lane: one 128-bit load per word row) and 4*BPW consecutive 32-row blocks;
// wave w takes BPW of them and issues all 3*BPW loads before converting.  The
// activations of the workgroup's rows are staged in LDS in the order the
// code pairs come out (see q3_block_pairs).  Partial sums are reduced across
// waves in LDS and across the S workgroups of a tile through the workspace.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

template <bool F16, int BPW>
__global__ __launch_bounds__(kThreads) void q3_matvec_kernel(
    const void* __restrict__ xv, const uint32_t* __restrict__ qw, const void* __restrict__ sv,
    const void* __restrict__ zv, void* __restrict__ yv, float* __restrict__ part,
    unsigned* __restrict__ counters, int K, int N, int S) {
  constexpr int BPG = 4 * BPW;  // blocks per workgroup
  constexpr int XW = F16 ? 1 : 2;
  __shared__ uint32_t xp[BPG][16][XW];
  __shared__ float red[4][kTileN + 4];
  __shared__ float xsum_w[4];
  __shared__ int last_flag;

  const int nb = K / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ct = blockIdx.x / S, s = blockIdx.x % S;
  const int blk0 = s * BPG;
  const int col0 = ct * kTileN + lane * 4;
  const bool col_ok = col0 < N;

  // 1. Stream this wave's blocks: 3 word rows each, 4 columns per lane.
  //    Blocks past the end fall outside the buffer and read as zero.
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(qw, 3 * nb * N * 4);
  u32x4 w[BPW][3];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int blk = blk0 + wave * BPW + i;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      w[i][j] = buffer_stream(wr, col_ok ? ((3 * blk + j) * N + col0) * 4 : kOutOfRange);
  }

  // 2. Stage x for these blocks in pair order, and form sum_k x[k].
  float my_sum = 0.0f;
  for (int idx = tid; idx < BPG * 16; idx += kThreads) {
    const int bl = idx >> 4, P = idx & 15;
    const int blk = blk0 + bl;
    const int ka = 32 * blk + q3_pair(P).a, kb = 32 * blk + q3_pair(P).b;
    if constexpr (F16) {
      const _Float16* x = reinterpret_cast<const _Float16*>(xv);
      _Float16 a = 0, b = 0;
      if (blk < nb) { a = x[ka]; b = x[kb]; }
      xp[bl][P][0] = as_u32((h2){a, b});
      my_sum += (float)a + (float)b;
    } else {
      const float* x = reinterpret_cast<const float*>(xv);
      float a = 0.0f, b = 0.0f;
      if (blk < nb) { a = x[ka]; b = x[kb]; }
      xp[bl][P][0] = __builtin_bit_cast(uint32_t, a);
      xp[bl][P][1] = __builtin_bit_cast(uint32_t, b);
      my_sum += a + b;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) my_sum += __shfl_xor(my_sum, o);
  if (lane == 0) xsum_w[wave] = my_sum;
  __syncthreads();
  const float xsum = (xsum_w[0] + xsum_w[1]) + (xsum_w[2] + xsum_w[3]);

  // 3. Exact codes times x, accumulated in fp32.
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int bl = wave * BPW + i;
    uint32_t xr[16][XW];
#pragma unroll
    for (int P = 0; P < 16; ++P)
#pragma unroll
      for (int t = 0; t < XW; ++t) xr[P][t] = xp[bl][P][t];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      h2 pr[16];
      q3_block_pairs(w[i][0][c], w[i][1][c], w[i][2][c], pr);
#pragma unroll
      for (int P = 0; P < 16; ++P) {
        if constexpr (F16) {
          acc[c] = dot2(pr[P], as_h2(xr[P][0]), acc[c]);
        } else {
          acc[c] = __builtin_fmaf((float)pr[P].x, __builtin_bit_cast(float, xr[P][0]), acc[c]);
          acc[c] = __builtin_fmaf((float)pr[P].y, __builtin_bit_cast(float, xr[P][1]), acc[c]);
        }
      }
    }
  }

  // 4. Across waves; thread t owns column t of the tile.
#pragma unroll
  for (int c = 0; c < 4; ++c) red[wave][lane * 4 + c] = acc[c];
  __syncthreads();
  const int n = ct * kTileN + tid;
  const float A = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
  float val = 0.0f;
  if (n < N) {
    float sc, ze;
    if constexpr (F16) {
      sc = (float)reinterpret_cast<const _Float16*>(sv)[n];
      ze = (float)reinterpret_cast<const _Float16*>(zv)[n];
    } else {
      sc = reinterpret_cast<const float*>(sv)[n];
      ze = reinterpret_cast<const float*>(zv)[n];
    }
    val = sc * A - ze * xsum;
  }

  auto store = [&](float v) {
    if constexpr (F16) reinterpret_cast<_Float16*>(yv)[n] = (_Float16)v;
    else reinterpret_cast<float*>(yv)[n] = v;
  };
  if (S == 1) {
    if (n < N) store(val);
    return;
  }
  if (n < N) part[(size_t)s * N + n] = val;
  if (splitk_arrive(&counters[ct], S, &last_flag)) {
    if (n < N) {
      float t = 0.0f;
      for (int j = 0; j < S; ++j) t += part[(size_t)j * N + n];
      store(t);
    }
    splitk_reset(&counters[ct]);
  }
}

// Blocks per wave: the most (loads in flight per lane) that still gives
// enough workgroups to cover the GPU.
SplitPlan plan_q3(int K, int N) {
  SplitPlan p;
  p.mt = 1;
  p.n_tiles = (N + kTileN - 1) / kTileN;
  const int nb = K / 32;
  int bpw = 1;
  for (int cand : {4, 2, 1}) {
    const int S = (nb + 4 * cand - 1) / (4 * cand);
    if (p.n_tiles * S >= 240 || cand == 1) { bpw = cand; break; }
  }
  const int ov = env_unit_override();
  if (ov == 1 || ov == 2 || ov == 4 || ov == 8) bpw = ov;
  p.unit = bpw;
  p.splits = (nb + 4 * bpw - 1) / (4 * bpw);
  return p;
}

template <bool F16, int BPW>
static hipError_t launch_q3_t(const void* x, const int32_t* qw, const void* scales,
                              const void* zeros, void* y, int K, int N, const SplitPlan& p,
                              void* ws, hipStream_t s) {
  unsigned* counters = reinterpret_cast<unsigned*>(ws);
  float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + ws_counter_bytes(p.n_tiles));
  hipLaunchKernelGGL((q3_matvec_kernel<F16, BPW>), dim3(p.n_tiles * p.splits), dim3(kThreads), 0,
                     s, x, reinterpret_cast<const uint32_t*>(qw), scales, zeros, y, part, counters,
                     K, N, p.splits);
  return hipGetLastError();
}

template <bool F16>
static hipError_t launch_q3_f(const void* x, const int32_t* qw, const void* scales,
                              const void* zeros, void* y, int K, int N, const SplitPlan& p,
                              void* ws, hipStream_t s) {
  switch (p.unit) {
    case 1: return launch_q3_t<F16, 1>(x, qw, scales, zeros, y, K, N, p, ws, s);
    case 2: return launch_q3_t<F16, 2>(x, qw, scales, zeros, y, K, N, p, ws, s);
    case 4: return launch_q3_t<F16, 4>(x, qw, scales, zeros, y, K, N, p, ws, s);
    default: return launch_q3_t<F16, 8>(x, qw, scales, zeros, y, K, N, p, ws, s);
  }
}

hipError_t launch_q3(const void* x, const int32_t* qw, const void* scales, const void* zeros,
                     void* y, int K, int N, bool f16, const SplitPlan& p, void* ws,
                     hipStream_t s) {
  return f16 ? launch_q3_f<true>(x, qw, scales, zeros, y, K, N, p, ws, s)
             : launch_q3_f<false>(x, qw, scales, zeros, y, K, N, p, ws, s);
}

}  // namespace wq
