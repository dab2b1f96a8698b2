// 4-bit group-wise GEMM for more rows of X (9 .. 64 per launch), reading the
// packed weight once per launch.
//
//   Y[m, n] = sum_g scale[g, n] * sum_{rows i of group g} X[m, perm[i]] * (u[i, n] - z[g, n])
//
// with z = 8 for the symmetric codes, or the stored zero point ("Quantization
// CUDA", tom-jerr.github.io: "Int4 Weight Only Quantization", "量化粒度"
// (x = S (q - Z), groups of 128 along K), "Marlin 格式" (the offline
// re-layout, (W_int4 - Zero) * Scale); "GPTQ算法解析", intelliparadigm.com,
// section 4.1: act_order).  The packed weight is the one wq_prepack_q4
// writes for the small-M kernel: rows in group order, panels of 16 columns,
// blocks of 128 rows in matrix-core operand order, and the row tables.
//
// Two launches.
// (1) Gather: X goes once per call into a caller workspace, in the packed
//     weight's row order and already in matrix-core operand order: for MFMA
//     step s (32 rows) and 16-row tile mb the 16 x 32 operand is 1 KB, lane
//     l's 16 bytes holding row 16 mb + l % 16, group-order rows
//     32 s + 8 (l / 16) .. +7 in the order 0 4 1 5 2 6 3 7 (the order of the
//     codes in a packed word).  Each lane reads its 8 original row numbers
//     from the forward row table and gathers the 8 values, so every operand
//     block is written whole by one wave.  Rows of X past M and padding rows
//     past K are zero.  The same launch writes the sums of X over runs of R
//     group-order rows (R = 64, or 32 for groups of 32), times the offset's
//     factor: S = -8 * 2^-24 * sum for the symmetric codes, 2^-24 * sum with
//     zero points.
// (2) The GEMM.  A workgroup takes a run of at most 3 panels and every row
//     of the launch (one to four 16-row tiles).  K is cut into units of 64
//     rows (two MFMA steps); each of the 8 waves walks a contiguous range of
//     whole blocks on its own, with a ring of RD units in flight: per unit
//     its X operands (1 KB per tile and step, contiguous), its weights
//     (8 bytes per lane and panel), the row sums and the scales.  Every
//     operand and table is read through a buffer range that ends where the
//     wave's share ends, so the loads the ring issues past it return zeros
//     and cost no memory traffic; no LDS and no barrier until the end.  A
//     weight word, unpacked into an operand, feeds one MFMA per 16-row tile.
//     The accumulation of each run starts from the offset term instead of
//     zero:
//       C = S' + 2^-24 * sum_i x_i u_i = 2^-24 * sum_i x_i (u_i - z),
//     S' = S (symmetric) or -z * S (zero points), and closes with
//       tot += scale * C.
//     At the end the 8 waves' partial tiles are added in LDS in a fixed order
//     and Y = 2^24 * tot.
#include "q4_layout.hpp"
#include "wq_internal.h"

namespace wq {

constexpr int kQTThreads = 512;
constexpr int kQTWaves = kQTThreads / 64;
constexpr int kQTMaxRun = 3;    // panels per workgroup at most
constexpr int kQTMaxRows = 64;  // rows of X per launch at most

int q4_tiled_kp(int K) { return (K + kQ4Block - 1) / kQ4Block * kQ4Block; }

// Workspace: the operand-order copy of X (mbt 16-row tiles of Kp halves
// each), then the row sums S: [Kp / R][mbt * 16] fp32, sized for R = 32.
static size_t q4_xo_bytes(int mbt, int Kp) { return (size_t)mbt * 16 * Kp * 2; }
size_t q4_tiled_workspace_bytes(int M, int K) {
  if (M <= kQ4TiledMinRows) return 0;
  const int mbt = (M + 15) / 16, Kp = q4_tiled_kp(K);
  return q4_xo_bytes(mbt, Kp) + (size_t)(Kp / 32) * mbt * 16 * 4;
}

// (1) Workgroup (unit u of 64 group-order rows, tile mb); wave h builds the
// operand block of step 2u + h.  R64: one sum per unit (both waves), else
// one per step.  zs: the factor the sums are stored with.
constexpr int kQXThreads = 128;
__global__ __launch_bounds__(kQXThreads) void q4_xgather_kernel(const _Float16* __restrict__ X,
                                                                const uint16_t* __restrict__ fwd,
                                                                _Float16* __restrict__ Xo,
                                                                float* __restrict__ S, int M, int K,
                                                                int mbt, int R64, float zs) {
  __shared__ float part[16];
  const int t = threadIdx.x, lane = t & 63, h = t >> 6;
  const int u = blockIdx.x, mb = blockIdx.y;
  const int step = 2 * u + h;
  const int m = 16 * mb + (lane & 15);
  // Original rows of group-order rows 32 step + 8 (lane / 16) + e, e = 0..7
  // (0xFFFF: a padding row).
  const u32x4 tv = *reinterpret_cast<const u32x4*>(fwd + 32 * step + 8 * (lane >> 4));
  const uint16_t* xrow = reinterpret_cast<const uint16_t*>(X) + (size_t)m * K;
  uint32_t v[8];
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = (int)((tv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    v[e] = (m < M && k < K) ? (uint32_t)xrow[k] : 0u;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sum += (float)__builtin_bit_cast(_Float16, (uint16_t)v[e]);
  // Operand order 0 4 1 5 2 6 3 7: half 2 j holds row j, half 2 j + 1 row j + 4.
  const u32x4 o = {v[0] | (v[4] << 16), v[1] | (v[5] << 16), v[2] | (v[6] << 16),
                   v[3] | (v[7] << 16)};
  *reinterpret_cast<u32x4*>(Xo + (((size_t)step * mbt + mb) * 64 + lane) * 8) = o;
  // Rows of the step: the 4 lanes of row m hold 8 each.
  sum += __shfl_xor(sum, 16);
  sum += __shfl_xor(sum, 32);
  const size_t rows = (size_t)mbt * 16;
  if (R64) {
    if (h == 1 && lane < 16) part[lane] = sum;
    __syncthreads();
    if (h == 0 && lane < 16) S[(size_t)u * rows + m] = (sum + part[lane]) * zs;
  } else if (lane < 16) {
    S[(size_t)step * rows + m] = sum * zs;
  }
}

// (2) MB: 16-row tiles (M <= 16 MB); NCL: runs closed per unit (1 for groups
// of 64 rows or more, 2 for groups of 32); RD: units in flight per wave
// (even, so a unit's half of its weight block is known at compile time).
// lgu: log2 of the units per group (NCL = 1).
template <int MB, int NCL, bool ZP, int RD>
__global__ __launch_bounds__(kQTThreads) void q4_tiled_kernel(
    const _Float16* __restrict__ Xo, const float* __restrict__ S, const uint8_t* __restrict__ Wp,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ Y, int M, int mb0, int mbt, int N, int ngroups, int lgu, int nb,
    int npanels) {
  static_assert(RD % 2 == 0, "ring depth must be even");
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
  constexpr int MT = 16 * MB;
  __shared__ float red[kQTMaxRun * kQTWaves * MT * 16];  // [run][wave][MT][16]

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Each XCD (workgroups b = x mod 8) takes a contiguous range of panel runs,
  // so a 128-byte line of a scale or zero row (four panels) is fetched into
  // one XCD's L2.
  const int G8 = gridDim.x % 8 == 0 ? gridDim.x / 8 : 0;
  const int run = G8 ? (int)(blockIdx.x % 8) * G8 + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const int p_begin = (int)((long long)run * npanels / gridDim.x);
  const int npr = (int)((long long)(run + 1) * npanels / gridDim.x) - p_begin;
  // This wave's blocks [bw0, bw1) of every panel: units [2 bw0, 2 bw1).
  // The share a wave takes rotates with the workgroup, so the workgroups of
  // an XCD do not all read the same rows of X at the same moment.
  const int share = (wave + run) % kQTWaves;
  const int bw0 = share * nb / kQTWaves, bw1 = (share + 1) * nb / kQTWaves;
  const int nu = 2 * (bw1 - bw0);
  const int col = lane & 15;

  // Buffer ranges that end with this wave's share.
  const int xunit = 2 * mbt * 1024;  // X operand bytes of one unit, all tiles
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(reinterpret_cast<const char*>(Xo) + (size_t)2 * bw0 * xunit, nu * xunit);
  constexpr int CPU = NCL;                   // sum chunks per unit
  const int chunk = mbt * 16 * 4;            // bytes of one chunk of sums
  const __amdgpu_buffer_rsrc_t sr =
      make_rsrc(reinterpret_cast<const char*>(S) + (size_t)2 * bw0 * CPU * chunk, nu * CPU * chunk);
  __amdgpu_buffer_rsrc_t wr[kQTMaxRun];
#pragma unroll
  for (int p = 0; p < kQTMaxRun; ++p) {
    const int panel = p < npr ? p_begin + p : 0;
    wr[p] = make_rsrc(Wp + ((size_t)panel * nb + bw0) * 1024, p < npr ? (bw1 - bw0) * 1024 : 0);
  }
  const __amdgpu_buffer_rsrc_t scr = make_rsrc(scales, ngroups * N * 2);
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(ZP ? zeros : scales, ngroups * N * 2);
  int slane[kQTMaxRun];  // this lane's column in a scale row, or out of range
#pragma unroll
  for (int p = 0; p < kQTMaxRun; ++p) {
    const int n = (p_begin + p) * kQ4Panel + col;
    slane[p] = (p < npr && n < N) ? n * 2 : kOutOfRange;
  }
  const int xlane = lane * 16, wlane = lane * 16, sl = (lane >> 4) * 16;

  struct Unit {
    u32x4 a[2][MB];               // X operands: step s, tile mb
    u32x2v w[kQTMaxRun];          // weight words of steps 2 (u & 1), +1
    f4 s[NCL][MB];                // offset terms (row sums)
    uint32_t sc[kQTMaxRun][NCL];  // scale bits of the runs' groups
    uint32_t zq[kQTMaxRun][NCL];  // zero bits (ZP)
  };
  // Loads of this wave's unit j (ring slot parity P = j & 1).  The ring asks
  // for up to RD units past the wave's share; those loads take the share's
  // last unit again (their values are never used), so every address stays
  // inside the wave's ranges.  A wave with no share has empty ranges: its
  // loads all return zeros.
  auto load = [&](int jr, Unit& q, auto parity) {
    constexpr int P = decltype(parity)::value;
    const int j = jr < nu ? jr : (nu > 0 ? nu - 1 : 0);
    const int xo = j * xunit + mb0 * 1024;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        q.a[st][mb] = __builtin_amdgcn_raw_buffer_load_b128(xr, xlane + mb * 1024,
                                                            xo + st * mbt * 1024, 0);
    const int wo = (j >> 1) * 1024;
#pragma unroll
    for (int p = 0; p < kQTMaxRun; ++p)
      q.w[p] = __builtin_bit_cast(
          u32x2v, __builtin_amdgcn_raw_buffer_load_b64(wr[p], wlane + 8 * P, wo, 0));
#pragma unroll
    for (int k = 0; k < NCL; ++k)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        q.s[k][mb] = __builtin_bit_cast(
            f4, __builtin_amdgcn_raw_buffer_load_b128(sr, sl + (mb0 + mb) * 64,
                                                      (j * CPU + k) * chunk, 0));
    const int u = 2 * bw0 + j;
#pragma unroll
    for (int k = 0; k < NCL; ++k) {
      // Padding rows past K (zero in X) take the last group's scale.
      const int g0 = NCL == 1 ? (u >> lgu) : 2 * u + k;
      const int so = (g0 < ngroups ? g0 : ngroups - 1) * N * 2;
#pragma unroll
      for (int p = 0; p < kQTMaxRun; ++p) {
        q.sc[p][k] = __builtin_amdgcn_raw_buffer_load_b16(scr, slane[p], so, 0);
        if constexpr (ZP) q.zq[p][k] = __builtin_amdgcn_raw_buffer_load_b16(zr, slane[p], so, 0);
      }
    }
  };

  f4 tot[kQTMaxRun][MB];
#pragma unroll
  for (int p = 0; p < kQTMaxRun; ++p)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot[p][mb] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // One unit.  Every panel slot runs, also past the run (its weights and
  // scales read as zero, its tile is never stored): no branch between an
  // MFMA and the first read of its result.
  auto compute = [&](const Unit& q) {
    h8 b[2][kQTMaxRun];
#pragma unroll
    for (int p = 0; p < kQTMaxRun; ++p) {
      b[0][p] = __builtin_bit_cast(h8, q4_mfma_operand(q.w[p][0]));
      b[1][p] = __builtin_bit_cast(h8, q4_mfma_operand(q.w[p][1]));
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const h8 a[2] = {__builtin_bit_cast(h8, q.a[0][mb]), __builtin_bit_cast(h8, q.a[1][mb])};
#pragma unroll
      for (int p = 0; p < kQTMaxRun; ++p) {
#pragma unroll
        for (int k = 0; k < NCL; ++k) {
          f4 c = q.s[k][mb];
          if constexpr (ZP) c *= -(float)__builtin_bit_cast(_Float16, (uint16_t)q.zq[p][k]);
          if constexpr (NCL == 1) {
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b[0][p], c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b[1][p], c, 0, 0, 0);
          } else {
            c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[k], b[k][p], c, 0, 0, 0);
          }
          const float sv = (float)__builtin_bit_cast(_Float16, (uint16_t)q.sc[p][k]);
#pragma unroll
          for (int r = 0; r < 4; ++r) tot[p][mb][r] = __builtin_fmaf(sv, c[r], tot[p][mb][r]);
        }
      }
    }
  };

  // The ring: slot i holds unit j + i.  Loads are issued in unit order and
  // scheduling barriers keep them so, so the oldest slot's loads are always
  // the first outstanding ones and each wait before a compute covers only
  // its own unit.
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  Unit q[RD];
#pragma unroll
  for (int i = 0; i < RD; ++i) {
    if (i % 2 == 0) load(i, q[i], P0{});
    else load(i, q[i], P1{});
    __builtin_amdgcn_sched_barrier(0);
  }
  int j = 0;
  for (; j + RD < nu; j += RD) {
#pragma unroll
    for (int i = 0; i < RD; ++i) {
      compute(q[i]);
      if (i % 2 == 0) load(j + RD + i, q[i], P0{});
      else load(j + RD + i, q[i], P1{});
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < RD; ++i)
    if (j + i < nu) compute(q[i]);

#pragma unroll
  for (int p = 0; p < kQTMaxRun; ++p)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * mb + 4 * (lane >> 4) + r;
        red[((p * kQTWaves + wave) * MT + m) * 16 + col] = tot[p][mb][r];
      }
  __syncthreads();
  for (int r = t; r < npr * MT * 16; r += kQTThreads) {
    const int pi = r / (MT * 16), m = (r / 16) % MT, c = r % 16;
    const int n = (p_begin + pi) * kQ4Panel + c;
    const float* v = red + (pi * kQTWaves * MT + m) * 16 + c;
    float sum = 0.0f;
#pragma unroll
    for (int w2i = 0; w2i < kQTWaves; ++w2i) sum += v[w2i * MT * 16];
    if (m < M && n < N) Y[(size_t)m * N + n] = (_Float16)(sum * kTwo24);
  }
}

// Units in flight per wave: as many as fit the registers without spilling.
constexpr int q4_tiled_depth(int MB, int NCL, bool ZP) {
  return NCL == 1 ? (MB == 1 ? 6 : MB == 2 ? 4 : 2) : (MB == 1 ? 4 : 2);
}

template <int MB, int NCL, bool ZP>
static hipError_t launch_q4_tiled_t(const _Float16* Xo, const float* S, const uint8_t* Wp,
                                    const _Float16* scales, const _Float16* zeros, _Float16* Y,
                                    int M, int mb0, int mbt, int K, int N, int G, hipStream_t s) {
  constexpr int RD = q4_tiled_depth(MB, NCL, ZP);
  const int nb = q4_tiled_kp(K) / kQ4Block, npanels = (N + kQ4Panel - 1) / kQ4Panel;
  const int cus = device_cus();
  int grid = npanels < cus ? npanels : cus;
  if ((npanels + grid - 1) / grid > kQTMaxRun) grid = (npanels + kQTMaxRun - 1) / kQTMaxRun;
  int lgu = 0;
  while ((64 << lgu) < G) ++lgu;
  hipLaunchKernelGGL((q4_tiled_kernel<MB, NCL, ZP, RD>), dim3(grid), dim3(kQTThreads), 0, s, Xo, S,
                     Wp, scales, zeros, Y, M, mb0, mbt, N, K / G, lgu, nb, npanels);
  return hipGetLastError();
}

template <int MB>
static hipError_t launch_q4_tiled_mb(const _Float16* Xo, const float* S, const uint8_t* Wp,
                                     const _Float16* scales, const _Float16* zeros, _Float16* Y,
                                     int M, int mb0, int mbt, int K, int N, int G, hipStream_t s) {
  if (G == 32) {
    // Launches for groups of 32 take at most three tiles (see below).
    if constexpr (MB > 3) return hipErrorInvalidValue;
    else
      return zeros ? launch_q4_tiled_t<MB, 2, true>(Xo, S, Wp, scales, zeros, Y, M, mb0, mbt, K, N,
                                                    G, s)
                   : launch_q4_tiled_t<MB, 2, false>(Xo, S, Wp, scales, zeros, Y, M, mb0, mbt, K,
                                                     N, G, s);
  }
  return zeros ? launch_q4_tiled_t<MB, 1, true>(Xo, S, Wp, scales, zeros, Y, M, mb0, mbt, K, N, G, s)
               : launch_q4_tiled_t<MB, 1, false>(Xo, S, Wp, scales, zeros, Y, M, mb0, mbt, K, N, G,
                                                 s);
}

hipError_t launch_q4_tiled(const void* X, const void* packed, const void* scales,
                           const void* zeros, void* Y, void* ws, int M, int K, int N, int G,
                           hipStream_t s) {
  const int Kp = q4_tiled_kp(K);
  const int mbt = (M + 15) / 16;
  const uint8_t* Wp = reinterpret_cast<const uint8_t*>(packed);
  const uint16_t* fwd = reinterpret_cast<const uint16_t*>(Wp + q4_fwd_table_offset(K, N));
  _Float16* Xo = reinterpret_cast<_Float16*>(ws);
  float* S = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + q4_xo_bytes(mbt, Kp));
  const float zs = zeros ? 1.0f / kTwo24 : -8.0f / kTwo24;
  hipLaunchKernelGGL(q4_xgather_kernel, dim3(Kp / 64, mbt), dim3(kQXThreads), 0, s,
                     reinterpret_cast<const _Float16*>(X), fwd, Xo, S, M, K, mbt, G >= 64 ? 1 : 0,
                     zs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const _Float16* sc = reinterpret_cast<const _Float16*>(scales);
  const _Float16* zp = reinterpret_cast<const _Float16*>(zeros);
  // Groups of 32 close twice per unit; with four tiles that no longer fits
  // the registers, so those launches take at most 48 rows.
  const int rows = G == 32 ? 48 : kQTMaxRows;
  for (int m0 = 0; m0 < M; m0 += rows) {
    const int mc = M - m0 < rows ? M - m0 : rows;
    _Float16* Yc = reinterpret_cast<_Float16*>(Y) + (size_t)m0 * N;
    const int mb0 = m0 / 16;
    switch ((mc + 15) / 16) {
      case 1: e = launch_q4_tiled_mb<1>(Xo, S, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
      case 2: e = launch_q4_tiled_mb<2>(Xo, S, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
      case 3: e = launch_q4_tiled_mb<3>(Xo, S, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
      default: e = launch_q4_tiled_mb<4>(Xo, S, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
