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
// into column pairs: pair q (columns 2q, 2q + 1) is K/8 contiguous 16-byte
// pieces, piece b holding rows 8b .. 8b + 7.  Word d of a piece holds rows
// 2d and 2d + 1 of column 2q in bytes 0 and 1, and the same rows of column
// 2q + 1 in bytes 2 and 3, so one v_perm_b32 puts a column's two rows into
// an fp16 pair (q8_col_pair).  Codes are stored biased (u = q + 128): the
// bias is removed with one sum of x per piece, and the biased byte goes
// straight into an fp16 mantissa as a subnormal, u * 2^-24, so every
// product x * u * 2^-24 is exact in fp32.
//
// The product.  A wave owns one column pair over all of K, so no partial sum
// ever leaves the wave: at step i lane l takes piece 64 i + l of its pair
// (the wave reads 1 KB of contiguous memory per step), and one cross-lane
// reduction at the end gives the two outputs.  Eight waves (a 16-column
// panel) share the activations, staged once per 4096 rows in LDS.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// 512 threads (8 wave64s, two per SIMD): while one wave of a SIMD converts
// its codes the other's loads are still landing.
constexpr int kQ8Threads = 512;
constexpr int kQ8Steps = 8;                    // pieces per lane per chunk
constexpr int kQ8Chunk = 64 * kQ8Steps * 8;    // rows of K per chunk: 4096
// From this many rows of X on, the product runs as a tiled matrix-core GEMM
// (q8_gemm.hip) instead of one streaming pass over the weight per 8 rows.
constexpr int kQ8GemmMinRows = 9;

// Panel plan: 16-column panels (8 column pairs); u = pieces per pair.
PanelPlan plan_q8(int K, int N) {
  PanelPlan p{};
  p.P = 16;
  p.cpp = 1;
  p.npanels = N / 16;
  p.u = K / 8;
  p.nsa = 0;
  p.packed_bytes = (size_t)K * N;
  return p;
}

// ---------------------------------------------------------------------------
// Offline re-layout: one thread per 16-byte piece (pair q, rows 8b .. 8b + 7).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q8_prepack_kernel(const int8_t* __restrict__ W,
                                                              uint32_t* __restrict__ out, int K,
                                                              int N) {
  const int KB = K / 8;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)(N / 2) * KB) return;
  const int q = (int)(idx / KB), b = (int)(idx % KB);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(W) + (size_t)8 * b * N + 2 * q;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t r0 = *reinterpret_cast<const uint16_t*>(src + (size_t)(2 * d) * N);
    const uint32_t r1 = *reinterpret_cast<const uint16_t*>(src + (size_t)(2 * d + 1) * N);
    // bytes: row 2d col 0, row 2d+1 col 0, row 2d col 1, row 2d+1 col 1
    const uint32_t v = (r0 & 0xFFu) | ((r1 & 0xFFu) << 8) | ((r0 >> 8) << 16) | ((r1 >> 8) << 24);
    out[idx * 4 + d] = v ^ 0x80808080u;
  }
}

// ---------------------------------------------------------------------------
// The fused product, MT rows of X per pass.
// ---------------------------------------------------------------------------
// FOLD (one or two rows of X, G a power of two >= 128, log2 G = gsh): the
// 16 lanes of a quarter-wave hold 128 consecutive rows at every step, i.e.
// part of one group, so a quarter needs 16 scales per 4096 rows (8 steps x 2
// columns).  Lane j of the quarter loads the one of step j / 2, column j % 2
// (one 4-byte load per lane), and DPP row broadcasts hand all 16 to every
// lane of the quarter as soon as it lands, before the weights.  Otherwise
// each piece's two sums take their scales (one 8-byte load per piece).
// u = q + 128: both columns of a piece start at -128 * sum(x) over the
// piece's 8 activations, in 2^-24 units.
__device__ __forceinline__ float q8_piece_bias(const u32x4 x) {
  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  float s = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) s = dot2(as_h2(x[d]), ones, s);
  return s * (-128.0f / kTwo24);
}

// x from lane (l + R) mod 16 of this lane's 16-lane row (DPP row_ror:R).
template <int R>
__device__ __forceinline__ float q8_row_rotate(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + R, 0xF, 0xF, true));
}

// Lane J of each 16-lane row, to every lane of the row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float q8_row_share(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + J, 0xF, 0xF, true));
}
// s[j] = lane j's value of this lane's 16-lane row, j = 0 .. 15.
template <int J = 0>
__device__ __forceinline__ void q8_row_all(float x, float (&s)[2 * kQ8Steps]) {
  if constexpr (J < 2 * kQ8Steps) {
    s[J] = q8_row_share<J>(x);
    q8_row_all<J + 1>(x, s);
  }
}

template <int MT, bool FOLD>
__global__ __launch_bounds__(kQ8Threads) void q8_pair_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const float* __restrict__ scales, _Float16* __restrict__ Y, int M, int K, int N, int G,
    int gsh) {
  __shared__ u32x4 xs[MT][kQ8Threads];  // rows r0 .. r0 + 4095 of the MT rows of X
  // The sums of x that remove the code bias.  FOLD (all 16 pieces a quarter
  // holds at a step share one group and so one scale): one sum per 128-row
  // block, formed once per workgroup while x is staged (the 16 staging lanes
  // of a block add their pieces' sums across the row) and read by every
  // wave; each lane of the quarter adds a sixteenth of it, exactly, so the
  // wave's reduction restores the whole.  Otherwise, with several rows of X,
  // each piece's sum is formed once by the thread that stages it (at one row
  // the per-piece sums are cheaper inside each wave).
  constexpr bool GS = FOLD;
  constexpr bool XB = MT > 1 && !FOLD;
  __shared__ float xb[XB ? MT : 1][kQ8Threads];  // -128 * 2^-24 * (sum of a piece's 8 x)
  // -128 * 2^-24 / 16 * (sum of x over 128-row block 4 i + j of the chunk)
  // at [m][j][i]: quarter j reads its 8 steps' values contiguously.
  __shared__ float gs[GS ? MT : 1][4][kQ8Steps];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Workgroups b and b + 8 run on the same XCD (dispatch is round-robin over
  // the 8 XCDs).  When the panel count allows, they take neighbouring panels,
  // which share the 128-byte lines of the fp32 scale rows, so each line is
  // fetched into one XCD's L2 only.
  const int bid = blockIdx.x;
  const int panel = (gridDim.x % 16 == 0) ? (bid & ~15) + 2 * (bid & 7) + ((bid >> 3) & 1) : bid;
  const int q = panel * 8 + wave;  // this wave's column pair
  const int KB = K / 8;            // pieces per pair

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, K * N);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (K / G) * N * 4);

  float tot[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m) tot[m][0] = tot[m][1] = 0.0f;

  for (int r0 = 0; r0 < K; r0 += kQ8Chunk) {
    const int b0 = r0 / 8;
    // Activations first (rows r0 + 8t .. + 7; zero past K and for m >= M),
    // then the scales, then the weight stream, so waiting for the activations
    // leaves the rest in flight.
    u32x4 xg[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xg[m] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, (m < M && r0 + 8 * t < K) ? (m * K + r0 + 8 * t) * 2 : kOutOfRange, 0, 0);
    constexpr int NS = FOLD ? 1 : kQ8Steps;  // scale loads per lane per chunk
    float fs = 0.0f;
    u32x2 sc[NS];
    if constexpr (FOLD) {
      // Lane l's scale: step (l % 16) / 2, column l % 2, the group of rows
      // r0 + 512 step + 128 (l / 16) .. + 127.
      const int row = r0 + 512 * ((lane & 15) >> 1) + 128 * (lane >> 4);
      fs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         sr, row < K ? ((row >> gsh) * N + 2 * q + (lane & 1)) * 4 : kOutOfRange,
                                         0, 0));
    } else {
#pragma unroll
      for (int i = 0; i < kQ8Steps; ++i) {
        const int b = b0 + 64 * i + lane;
        sc[i] = __builtin_amdgcn_raw_buffer_load_b64(
            sr, b < KB ? (((8 * b) / G) * N + 2 * q) * 4 : kOutOfRange, 0, 0);
      }
    }
    u32x4 w[kQ8Steps];
#pragma unroll
    for (int i = 0; i < kQ8Steps; ++i) {
      const int b = b0 + 64 * i + lane;
      w[i] = buffer_stream(wr, b < KB ? (q * KB + b) * 16 : kOutOfRange);
    }
    wait_vmcnt<kQ8Steps + NS>();  // the activations have landed
    if (r0 > 0) lds_barrier();     // every wave is done with the previous chunk
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      xs[m][t] = xg[m];
      if constexpr (XB) xb[m][t] = q8_piece_bias(xg[m]);
      if constexpr (GS) {
        // Piece t lies in block t / 16: the 16 lanes of a row (fixed order).
        float ps = q8_piece_bias(xg[m]) * (1.0f / 16.0f);
        ps += q8_row_rotate<8>(ps);
        ps += q8_row_rotate<4>(ps);
        ps += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, ps), 0x4E, 0xF, 0xF, true));
        ps += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, ps), 0xB1, 0xF, 0xF, true));
        if ((t & 15) == 0) gs[m][(t >> 4) & 3][t >> 6] = ps;
      }
    }
    lds_barrier();

    // The activations of every step and their piece sums first: they do
    // not wait for the weights.
    u32x4 xv[kQ8Steps][MT];
    float bias[kQ8Steps][MT];
#pragma unroll
    for (int i = 0; i < kQ8Steps; ++i)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        xv[i][m] = xs[m][64 * i + lane];
        if constexpr (XB) bias[i][m] = xb[m][64 * i + lane];
      }
    if constexpr (GS) {
#pragma unroll
      for (int i = 0; i < kQ8Steps; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) bias[i][m] = gs[m][lane >> 4][i];
    } else if constexpr (!XB) {
#pragma unroll
      for (int i = 0; i < kQ8Steps; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) bias[i][m] = q8_piece_bias(xv[i][m]);
    }
    // The quarter's 16 scales in every lane (FOLD): scale of step i,
    // column c at fsq[2i + c].
    float fsq[2 * kQ8Steps];
    if constexpr (FOLD) q8_row_all(fs, fsq);
#pragma unroll
    for (int i = 0; i < kQ8Steps; ++i) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float a0 = bias[i][m], a1 = bias[i][m];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          a0 = dot2(as_h2(q8_col_pair<0>(w[i][d])), as_h2(xv[i][m][d]), a0);
          a1 = dot2(as_h2(q8_col_pair<1>(w[i][d])), as_h2(xv[i][m][d]), a1);
        }
        const float s0 = FOLD ? fsq[2 * i] : as_f32(sc[i][0]);
        const float s1 = FOLD ? fsq[2 * i + 1] : as_f32(sc[i][1]);
        tot[m][0] = __builtin_fmaf(a0, s0, tot[m][0]);
        tot[m][1] = __builtin_fmaf(a1, s1, tot[m][1]);
      }
    }
  }

  {
    // Value j = 2m + c per lane, reduced over the whole wave.
    constexpr int V = 2 * MT;
    float r[V];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      r[2 * m] = tot[m][0];
      r[2 * m + 1] = tot[m][1];
    }
    bfly<V, 5, 0>(r, lane);
    bool owner;
    const int base = bfly_base<V, 0>(lane, owner);
    constexpr int LEFT = bfly_left<V, 0>();
    if (owner) {
#pragma unroll
      for (int j = 0; j < LEFT; ++j) {
        const int m = (base + j) >> 1, c = (base + j) & 1;
        if (m < M) Y[(size_t)m * N + 2 * q + c] = (_Float16)(r[j] * kTwo24);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Bit-exact check of the packed layout: every piece through q8_col_pair,
// written back as signed codes in [K, N].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q8_unpack_kernel(const uint8_t* __restrict__ Wp,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N) {
  const int KB = K / 8;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)(N / 2) * KB) return;
  const int q = (int)(idx / KB), b = (int)(idx % KB);
  const u32x4 w = *reinterpret_cast<const u32x4*>(Wp + idx * 16);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t c0 = q8_col_pair<0>(w[d]), c1 = q8_col_pair<1>(w[d]);
    const size_t row = (size_t)8 * b + 2 * d;
    codes[row * N + 2 * q] = (int8_t)((int)(c0 & 0xFFFFu) - 128);
    codes[(row + 1) * N + 2 * q] = (int8_t)((int)(c0 >> 16) - 128);
    codes[row * N + 2 * q + 1] = (int8_t)((int)(c1 & 0xFFFFu) - 128);
    codes[(row + 1) * N + 2 * q + 1] = (int8_t)((int)(c1 >> 16) - 128);
  }
}

hipError_t launch_q8_prepack(const int8_t* W, void* packed, int K, int N, hipStream_t s) {
  const size_t total = (size_t)(N / 2) * (K / 8);
  hipLaunchKernelGGL(q8_prepack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, W, reinterpret_cast<uint32_t*>(packed), K, N);
  return hipGetLastError();
}

hipError_t launch_q8_unpack(const void* packed, int8_t* codes, int K, int N, hipStream_t s) {
  const size_t total = (size_t)(N / 2) * (K / 8);
  hipLaunchKernelGGL(q8_unpack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint8_t*>(packed), codes, K, N);
  return hipGetLastError();
}

template <int MT, bool FOLD = false>
static hipError_t launch_q8_t(const void* X, const void* packed, const float* scales, void* Y,
                              int M, int K, int N, int G, hipStream_t s) {
  int gsh = 0;
  while ((1 << gsh) < G) ++gsh;
  hipLaunchKernelGGL((q8_pair_kernel<MT, FOLD>), dim3(N / 16), dim3(kQ8Threads), 0, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                     scales, reinterpret_cast<_Float16*>(Y), M, K, N, G, gsh);
  return hipGetLastError();
}

size_t q8_group_workspace_bytes(int M, int K, int N) {
  return M >= kQ8GemmMinRows ? q8_gemm_workspace_bytes(M, K, N) : 0;
}

hipError_t launch_q8_group(const void* X, const void* packed, const float* scales, void* Y,
                           void* ws, int M, int K, int N, int G, hipStream_t s) {
  if (M >= kQ8GemmMinRows && q8_gemm_supported(M, K, N, G))
    return launch_q8_gemm(X, packed, scales, Y, ws, M, K, N, G, s);
  // Rows of X beyond 8 run as further launches over the same weight.
  for (int m0 = 0; m0 < M; m0 += 8) {
    const int mc = (M - m0) < 8 ? (M - m0) : 8;
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)m0 * K * 2;
    void* Yc = reinterpret_cast<char*>(Y) + (size_t)m0 * N * 2;
    hipError_t e;
    const bool fold = G >= 128 && (G & (G - 1)) == 0;
    if (mc == 1)
      e = fold ? launch_q8_t<1, true>(Xc, packed, scales, Yc, mc, K, N, G, s)
               : launch_q8_t<1>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else if (mc == 2)
      e = fold ? launch_q8_t<2, true>(Xc, packed, scales, Yc, mc, K, N, G, s)
               : launch_q8_t<2>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else if (mc <= 4)  // per-piece scales: measured faster than the fold from 4 rows on
      e = launch_q8_t<4>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else
      e = launch_q8_t<8>(Xc, packed, scales, Yc, mc, K, N, G, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
