// Group-wise symmetric int8 weight-only GEMV / small-batch GEMM.
//
//   Y[m, n] = sum_g scale[g, n] * sum_{k in group g} X[m, k] * q[k, n]
//
// i.e. Y = X.(Wint*Sw) computed as (X.Wint)*Sw per group ("Quantization
// CUDA", tom-jerr.github.io, section "Int8 Weight Only Quantization"), with
// the int8 weight dequantised in registers as it streams in and never stored
// as floating point ("融合反量化与GEMM：LLM推理的CUDA内核优化实践",
// zingnex.cn, sections "核心优化思路" and "技术实现细节": one fp32 scale per 128
// rows of K per column).
//
// Layout.  The [K, N] weight is re-laid out once, offline (wq_prepack_q8),
// into column panels of P = 16*CPP columns.  A workgroup owns one panel over
// the whole of K, so no partial sum ever leaves the workgroup.  Inside a
// panel, thread t = s*CPP + c takes the 16 columns of chunk c and the u rows
// of slot s, in batches of 8 rows; the packed order puts the 16-byte piece
// that thread t reads at step i at ((panel*u + i) * active_threads + t) * 16,
// so every wave load is 1 KB of contiguous memory.  Codes are stored biased
// (u = q + 128): the bias is removed with one per-batch sum of x, and the
// biased byte goes straight into an fp16 mantissa as a subnormal (see
// q8_pairs_sub).
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// 512 threads (8 wave64s, two per SIMD): while one wave of a SIMD converts
// its codes the other's loads are still landing.
constexpr int kQ8Threads = 512;
constexpr int kQ8Batch = 8;  // rows per batch (never straddles a group: G % 32 == 0)
// From this many rows of X on, the product runs as a tiled matrix-core GEMM
// (q8_gemm.hip) instead of one streaming pass over the weight per 4 rows.
constexpr int kQ8GemmMinRows = 32;

// Panel plan: a pure function of (K, N); prepack and product agree on it.
PanelPlan plan_q8(int K, int N) {
  PanelPlan p{};
  p.P = (N % 32 == 0 && N / 32 >= 256) ? 32 : 16;
  p.cpp = p.P / 16;
  p.npanels = N / p.P;
  const int ns = kQ8Threads / p.cpp;
  p.u = kQ8Batch * ((K + kQ8Batch * ns - 1) / (kQ8Batch * ns));  // rows per slot
  p.nsa = (K + p.u - 1) / p.u;                                     // slots in use
  p.packed_bytes = (size_t)p.npanels * p.u * p.nsa * p.cpp * 16;
  return p;
}

// ---------------------------------------------------------------------------
// Offline re-layout: one thread per 16-byte output piece.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q8_prepack_kernel(const int8_t* __restrict__ W,
                                                              uint32_t* __restrict__ out, int K,
                                                              int N, PanelPlan p) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const int nta = p.nsa * p.cpp;
  const size_t total = (size_t)p.npanels * p.u * nta;
  if (idx >= total) return;
  const int t = (int)(idx % nta);
  const size_t pi = idx / nta;
  const int i = (int)(pi % p.u), panel = (int)(pi / p.u);
  const int s = t / p.cpp, c = t % p.cpp;
  const int row = s * p.u + i;
  const int col0 = panel * p.P + 16 * c;
  uint32_t v[4] = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};  // padding rows: q = 0
  if (row < K) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(W + (size_t)row * N + col0);
#pragma unroll
    for (int d = 0; d < 4; ++d) v[d] = src[d] ^ 0x80808080u;
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) out[idx * 4 + d] = v[d];
}

// ---------------------------------------------------------------------------
// The fused product.
// ---------------------------------------------------------------------------
// FOLD (M = 1, 16-column panels, 16 u == G): the 16 lanes of a quarter-wave
// hold the rows of one group, so their sums are reduced first and the
// group's scale is applied once per column on the reduced value: one 4-byte
// scale load per lane instead of four 16-byte loads, and one multiply.
template <int MT, int CPP, bool FOLD>
__global__ __launch_bounds__(kQ8Threads) void q8_panel_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const float* __restrict__ scales, _Float16* __restrict__ Y, int M, int K, int N, int G,
    int u, int nsa, int packed_bytes) {
  constexpr int P = 16 * CPP;
  constexpr int V = 16 * MT;                // results per chunk: [m][16 columns]
  constexpr int LOWBIT = CPP == 1 ? 0 : 1;  // lane bit 0 selects the chunk when CPP == 2
  constexpr int LEFT = bfly_left<V, LOWBIT>();
  constexpr int RB = kQ8Batch;
  static_assert(!FOLD || (MT == 1 && CPP == 1), "FOLD needs one row and 16-column panels");
  __shared__ float red[kQ8Threads / 64][CPP][V];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // Workgroups b and b + 8 run on the same XCD (dispatch is round-robin over
  // the 8 XCDs).  When the panel count allows, they take neighbouring panels,
  // which share the 128-byte lines of the fp32 scale rows, so each line is
  // fetched into one XCD's L2 only.
  const int bid = blockIdx.x;
  const int panel = (gridDim.x % 16 == 0) ? (bid & ~15) + 2 * (bid & 7) + ((bid >> 3) & 1) : bid;
  const int nta = nsa * CPP;
  const int c = t % CPP, s = t / CPP;
  const bool active = t < nta;
  const int col0 = panel * P + 16 * c;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, packed_bytes);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (K / G) * N * 4);
  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  float accT[MT][16];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) accT[m][j] = 0.0f;

  // FOLD: this lane's scale, group (s u) / G, column col0 + lane % 16.
  float fold_scale = 0.0f;
  if constexpr (FOLD) {
    const bool live0 = active && s * u < K;
    fold_scale = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(
                   sr, live0 ? (((s * u) / G) * N + col0 + (lane & 15)) * 4 : kOutOfRange, 0, 0));
  }

  const int nb = u / RB;
  for (int b = 0; b < nb; ++b) {
    const int row0 = s * u + RB * b;
    const bool live = active && row0 < K;
    // Activations of these 8 rows: one 128-bit load per row of X.
    u32x4 xv[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xv[m] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, (live && m < M) ? ((m * K + row0) * 2) : kOutOfRange, 0, 0);
    // The weight stream: 8 rows x 16 columns; 1 KB contiguous per wave load.
    u32x4 w[RB];
    const int wbase = ((panel * u + RB * b) * nta + t) * 16;
#pragma unroll
    for (int i = 0; i < RB; ++i) w[i] = buffer_stream(wr, active ? wbase + i * nta * 16 : kOutOfRange);
    f32x4 sc[4];
    if constexpr (!FOLD) {
      const int soff = live ? ((row0 / G) * N + col0) * 4 : kOutOfRange;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        sc[d] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(sr, soff + 16 * d, 0, 0));
    }

    // The codes are u = q + 128, so every column starts at -128 * sum(x),
    // in the 2^-24 units of the subnormal products.
    float acc[MT][16];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float xs = 0.0f;
#pragma unroll
      for (int q = 0; q < RB / 2; ++q) xs = dot2(as_h2(xv[m][q]), ones, xs);
      const float b0 = xs * (-128.0f / kTwo24);
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[m][j] = b0;
    }
#pragma unroll
    for (int q = 0; q < RB / 2; ++q) {  // row pair (2q, 2q + 1)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        h2 pr[4];
        q8_pairs_sub(w[2 * q][d], w[2 * q + 1][d], pr);
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int m = 0; m < MT; ++m)
            acc[m][4 * d + cc] = dot2(pr[cc], as_h2(xv[m][q]), acc[m][4 * d + cc]);
      }
    }
    // One group per batch: scale once (FOLD: after the reduction below).
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if constexpr (FOLD)
          accT[m][j] += acc[m][j];
        else
          accT[m][j] = __builtin_fmaf(acc[m][j], sc[j >> 2][j & 3], accT[m][j]);
      }
  }

  // Reduce over the slots of a chunk: the lanes of a wave, then the waves.
  float v[V];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 16; ++j) v[m * 16 + j] = accT[m][j];
  if constexpr (FOLD) {
    // Lane bits 3..0 first: lane l keeps column l % 16 of its quarter-wave's
    // group; scale it; then bits 5 and 4 add the wave's four groups.
    bfly<16, 3, 0>(v, lane);
    v[0] *= fold_scale;
    bfly<1, 5, 4>(v, lane);
    if (lane < 16) red[wave][0][lane] = v[0];
  } else {
    bfly<V, 5, LOWBIT>(v, lane);
    bool owner;
    const int base = bfly_base<V, LOWBIT>(lane, owner);
    if (owner) {
#pragma unroll
      for (int j = 0; j < LEFT; ++j) red[wave][c][base + j] = v[j];
    }
  }
  __syncthreads();
  for (int r = t; r < CPP * V; r += kQ8Threads) {
    const int rc = r / V, idx = r % V;
    const int m = idx / 16, col = panel * P + 16 * rc + (idx % 16);
    float sum = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kQ8Threads / 64; ++w2) sum += red[w2][rc][idx];
    if (m < M) Y[(size_t)m * N + col] = (_Float16)(sum * kTwo24);
  }
}

// ---------------------------------------------------------------------------
// Bit-exact check of the packed layout: rows (2q, 2q+1) of a slot go through
// q8_pairs_sub and are written back as signed codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q8_unpack_kernel(const uint8_t* __restrict__ Wp,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N, PanelPlan p) {
  const int nta = p.nsa * p.cpp;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)p.npanels * (p.u / 2) * nta;
  if (idx >= total) return;
  const int t = (int)(idx % nta);
  const size_t pi = idx / nta;
  const int q = (int)(pi % (p.u / 2)), panel = (int)(pi / (p.u / 2));
  const int s = t / p.cpp, c = t % p.cpp;
  const int row = s * p.u + 2 * q;
  const int col0 = panel * p.P + 16 * c;
  const u32x4 a = *reinterpret_cast<const u32x4*>(Wp + (((size_t)panel * p.u + 2 * q) * nta + t) * 16);
  const u32x4 b =
      *reinterpret_cast<const u32x4*>(Wp + (((size_t)panel * p.u + 2 * q + 1) * nta + t) * 16);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    h2 pr[4];
    q8_pairs_sub(a[d], b[d], pr);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const uint32_t bits = as_u32(pr[cc]);
      const int ua = (int)(bits & 0xFFFFu), ub = (int)(bits >> 16);
      const int col = col0 + 4 * d + cc;
      if (row < K) codes[(size_t)row * N + col] = (int8_t)(ua - 128);
      if (row + 1 < K) codes[(size_t)(row + 1) * N + col] = (int8_t)(ub - 128);
    }
  }
}

hipError_t launch_q8_prepack(const int8_t* W, void* packed, int K, int N, hipStream_t s) {
  const PanelPlan p = plan_q8(K, N);
  const size_t total = (size_t)p.npanels * p.u * p.nsa * p.cpp;
  hipLaunchKernelGGL(q8_prepack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, W, reinterpret_cast<uint32_t*>(packed), K, N, p);
  return hipGetLastError();
}

hipError_t launch_q8_unpack(const void* packed, int8_t* codes, int K, int N, hipStream_t s) {
  const PanelPlan p = plan_q8(K, N);
  const size_t total = (size_t)p.npanels * (p.u / 2) * p.nsa * p.cpp;
  hipLaunchKernelGGL(q8_unpack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint8_t*>(packed), codes, K, N,
                     p);
  return hipGetLastError();
}

template <int MT, int CPP, bool FOLD = false>
static hipError_t launch_q8_t(const void* X, const void* packed, const float* scales, void* Y,
                              int M, int K, int N, int G, const PanelPlan& p, hipStream_t s) {
  hipLaunchKernelGGL((q8_panel_kernel<MT, CPP, FOLD>), dim3(p.npanels), dim3(kQ8Threads), 0, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                     scales, reinterpret_cast<_Float16*>(Y), M, K, N, G, p.u, p.nsa,
                     (int)p.packed_bytes);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_q8_mt(const void* X, const void* packed, const float* scales, void* Y,
                               int M, int K, int N, int G, const PanelPlan& p, hipStream_t s) {
  if constexpr (MT == 1) {
    if (p.cpp == 1 && 16 * p.u == G)
      return launch_q8_t<1, 1, true>(X, packed, scales, Y, M, K, N, G, p, s);
  }
  return p.cpp == 1 ? launch_q8_t<MT, 1>(X, packed, scales, Y, M, K, N, G, p, s)
                    : launch_q8_t<MT, 2>(X, packed, scales, Y, M, K, N, G, p, s);
}

hipError_t launch_q8_group(const void* X, const void* packed, const float* scales, void* Y, int M,
                           int K, int N, int G, hipStream_t s) {
  if (M >= kQ8GemmMinRows && q8_gemm_supported(M, K, N, G))
    return launch_q8_gemm(X, packed, scales, Y, M, K, N, G, s);
  const PanelPlan p = plan_q8(K, N);
  // Rows of X beyond 4 run as further launches over the same panels (the
  // accumulators of 4 rows x 16 columns x 2 fill the register budget of a
  // 512-thread workgroup).
  for (int m0 = 0; m0 < M; m0 += 4) {
    const int mc = (M - m0) < 4 ? (M - m0) : 4;
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)m0 * K * 2;
    void* Yc = reinterpret_cast<char*>(Y) + (size_t)m0 * N * 2;
    hipError_t e;
    switch (mc) {
      case 1: e = launch_q8_mt<1>(Xc, packed, scales, Yc, mc, K, N, G, p, s); break;
      case 2: e = launch_q8_mt<2>(Xc, packed, scales, Yc, mc, K, N, G, p, s); break;
      default: e = launch_q8_mt<4>(Xc, packed, scales, Yc, mc, K, N, G, p, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
