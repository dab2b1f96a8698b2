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
// into tiles of 16 columns x 64 rows, 1 KB each: tile (p, b) holds columns
// 16p .. 16p + 15 and rows 64b .. 64b + 63 and sits at byte (p KT + b) 1024,
// KT = ceil(K / 64), so the tiles of a 16-column panel are contiguous.  Slot
// l of a tile (16 bytes at 16 l) holds column 16p + l % 16: bytes e = 0..7
// rows 64b + 8 (l / 16) + e, bytes 8 + e rows 64b + 32 + 8 (l / 16) + e.
// That is the matrix-core operand layout: a wave that reads a tile with one
// 16-byte load per lane holds in lane l the codes v_mfma_f32_16x16x32_f16
// takes for column l % 16 at k = 8 (l / 16) + e, for both 32-row steps of
// the tile.  Codes are stored biased (u = q + 128) so that a byte goes
// straight into an fp16 mantissa as the subnormal u 2^-24 (one v_perm_b32
// per two codes) and every product x u 2^-24 is exact in fp32; rows past K
// (K a multiple of 32 but not of 64) hold u = 128, i.e. q = 0.
//
// The product, up to 16 rows of X per launch.  A workgroup of 8 waves owns a
// panel; K is taken in chunks of 4096 rows, of which wave w takes the 8
// tiles 8w .. 8w + 7 (one 16-byte load each per lane, all issued at once).
// X is staged per chunk in LDS; the A operand of a step is 8 halves of one
// row of X (row l % 16 of the operand; at fewer rows, row 0 or zero rows).
// The offset 128 comes out per chain of steps inside one group: the staging
// threads form -128 2^-24 sum(x) over each chain's rows once per workgroup,
// and a chain's sums of x u 2^-24 take it before its scale:
// total += (chain sums - offset) * scale, in fp32, in units of 2^-24.  At the
// end the 8 waves' totals are added in a fixed order and rounded once to fp16.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

constexpr int kQ8Threads = 512;             // 8 wave64s, two per SIMD
constexpr int kQ8Waves = kQ8Threads / 64;
constexpr int kQ8Tiles = 8;                 // tiles per wave per chunk
constexpr int kQ8Steps = 2 * kQ8Tiles;      // 32-row steps per wave per chunk
constexpr int kQ8Chunk = kQ8Waves * kQ8Tiles * 64;  // rows of K per chunk: 4096
// LDS row of X: a chunk of fp16 plus 16 bytes, so that the 16 rows an
// operand read takes start on different banks.
constexpr int kQ8RowBytes = 2 * kQ8Chunk + 16;
// Rows of X per launch; from kQ8GemmMinRows rows on (groups a multiple of
// 64 rows) the tiled matrix-core GEMM (q8_gemm.hip) takes over.
constexpr int kQ8PassRows = 16;
constexpr int kQ8GemmMinRows = 17;

__host__ __device__ inline int q8_tiles_per_panel(int K) { return (K + 63) / 64; }

}  // namespace

// Panel plan: 16-column panels; u = tiles of 64 rows per panel.
PanelPlan plan_q8(int K, int N) {
  PanelPlan p{};
  p.P = 16;
  p.cpp = 1;
  p.npanels = N / 16;
  p.u = q8_tiles_per_panel(K);
  p.nsa = 0;
  p.packed_bytes = (size_t)p.npanels * p.u * 1024;
  return p;
}

// ---------------------------------------------------------------------------
// Offline re-layout: one thread per 16-byte slot.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q8_prepack_kernel(const int8_t* __restrict__ W,
                                                              uint8_t* __restrict__ out, int K,
                                                              int N) {
  const int KT = q8_tiles_per_panel(K);
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)(N / 16) * KT * 64) return;
  const int l = (int)(idx % 64);
  const size_t tile = idx / 64;
  const int b = (int)(tile % KT), p = (int)(tile / KT);
  const int col = 16 * p + (l & 15), h = l >> 4;
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t v = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 64 * b + 32 * (d >> 1) + 8 * h + 4 * (d & 1) + e;
      const uint32_t u = row < K ? ((uint32_t)(uint8_t)W[(size_t)row * N + col] ^ 0x80u) : 0x80u;
      v |= u << (8 * e);
    }
    w[d] = v;
  }
  *reinterpret_cast<u32x4*>(out + idx * 16) = (u32x4){w[0], w[1], w[2], w[3]};
}

// Bit-exact check of the packed layout: every slot through q8_byte_pair,
// written back as signed codes in [K, N].
__global__ __launch_bounds__(kThreads) void q8_unpack_kernel(const uint8_t* __restrict__ Wp,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N) {
  const int KT = q8_tiles_per_panel(K);
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)(N / 16) * KT * 64) return;
  const int l = (int)(idx % 64);
  const size_t tile = idx / 64;
  const int b = (int)(tile % KT), p = (int)(tile / KT);
  const int col = 16 * p + (l & 15), h = l >> 4;
  const u32x4 w = *reinterpret_cast<const u32x4*>(Wp + idx * 16);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t pr[2] = {q8_byte_pair<0>(w[d]), q8_byte_pair<1>(w[d])};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 64 * b + 32 * (d >> 1) + 8 * h + 4 * (d & 1) + e;
      if (row < K) codes[(size_t)row * N + col] = (int8_t)((int)((pr[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) - 128);
    }
  }
}

// ---------------------------------------------------------------------------
// The fused product.
// ---------------------------------------------------------------------------
namespace {

// DPP move of a float across lanes (full masks: every lane is written).
template <int CTRL>
__device__ __forceinline__ float q8_dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

}  // namespace

// MT: rows of X the launch stages (M <= MT; rows M .. MT - 1 are zero).
// CL: 32-row steps per chain, i.e. per scale.  A chain lies inside one group
// and inside one wave's 512 rows of a chunk: CL = G / 32 for groups of
// 32 .. 512 rows that are powers of two, 16 for larger powers of two (one
// chain per wave and chunk), 1 for other group sizes (a scale per step).
template <int MT, int CL>
__global__ __launch_bounds__(kQ8Threads) void q8_mfma_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const float* __restrict__ scales, _Float16* __restrict__ Y, int M, int K, int N, int G,
    int KT) {
  constexpr int NC = kQ8Steps / CL;            // chains per wave per chunk
  constexpr int NG = kQ8Chunk / (32 * CL);     // chains per chunk
  constexpr int RR = MT < 4 ? MT : 4;          // accumulator rows that can hold rows of X
  static_assert(CL == 1 || CL == 2 || CL == 4 || CL == 8 || CL == 16, "chain length");
  __shared__ __attribute__((aligned(16))) unsigned char xs[MT * kQ8RowBytes];  // the chunk of X
  __shared__ float cs[NG][16];  // [chain][row of X]: -128 2^-24 sum of x over the chain's rows
  __shared__ float red[kQ8Waves][MT][16];

  const int t = threadIdx.x, lane = t & 63, h = lane >> 4, j = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Workgroups b and b + 8 run on the same XCD (dispatch is round-robin over
  // the 8 XCDs).  When the panel count allows, they take neighbouring panels,
  // which share the 128-byte lines of the fp32 scale rows, so each line is
  // fetched into one XCD's L2 only.
  const int bid = blockIdx.x;
  const int panel = (gridDim.x % 16 == 0) ? (bid & ~15) + 2 * (bid & 7) + ((bid >> 3) & 1) : bid;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, (N / 16) * KT * 1024);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (K / G) * N * 4);

  // tot[r]: row 4 (l / 16) + r of X, column 16 panel + l % 16, units of 2^-24.
  float tot[RR];
#pragma unroll
  for (int r = 0; r < RR; ++r) tot[r] = 0.0f;
  const int arow = (MT > 1 && j < MT) ? j : 0;  // row of X in this lane's A operand

  for (int r0 = 0; r0 < K; r0 += kQ8Chunk) {
    // Activations first (rows r0 + 8t .. + 7; zero past K and for m >= M),
    // then the scales, then the weight tiles, so waiting for the activations
    // leaves the rest in flight.
    u32x4 xg[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xg[m] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, (m < M && r0 + 8 * t < K) ? (m * K + r0 + 8 * t) * 2 : kOutOfRange, 0, 0);
    float sc[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int row = r0 + 512 * wave + 32 * CL * c;
      sc[c] = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
          sr, row < K ? ((row / G) * N + 16 * panel + j) * 4 : kOutOfRange, 0, 0));
    }
    u32x4 wv[kQ8Tiles];
#pragma unroll
    for (int i = 0; i < kQ8Tiles; ++i) {
      const int b = r0 / 64 + kQ8Tiles * wave + i;
      wv[i] = buffer_stream(wr, b < KT ? (panel * KT + b) * 1024 + 16 * lane : kOutOfRange);
    }
    wait_vmcnt<NC + kQ8Tiles>();  // the activations have landed
    if (r0 > 0) lds_barrier();     // every wave is done with the previous chunk
    // Stage X; the chain sums: thread t's 8 rows lie in chain t / (4 CL),
    // whose 4 CL threads are consecutive lanes (fixed-order DPP sums).
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      *reinterpret_cast<u32x4*>(xs + m * kQ8RowBytes + 16 * t) = xg[m];
      const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
      float ps = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) ps = dot2(as_h2(xg[m][d]), ones, ps);
      ps *= -128.0f / kTwo24;
      ps += q8_dpp<0xB1>(ps);                        // quad_perm 1 0 3 2
      ps += q8_dpp<0x4E>(ps);                        // quad_perm 2 3 0 1
      if constexpr (CL >= 2) ps += q8_dpp<0x12C>(ps);  // row_ror:12, lane l + 4
      if constexpr (CL >= 4) ps += q8_dpp<0x128>(ps);  // row_ror:8
      if constexpr (CL >= 8) ps += __shfl_xor(ps, 16);
      if constexpr (CL >= 16) ps += __shfl_xor(ps, 32);
      if ((t & (4 * CL - 1)) == 0) cs[t / (4 * CL)][m] = ps;
    }
    lds_barrier();

    // Every step's A operand before any weight is waited for (the
    // scheduling barrier keeps the compiler from sinking the reads).
    h8 av[kQ8Steps];
#pragma unroll
    for (int st = 0; st < kQ8Steps; ++st)
      av[st] = *reinterpret_cast<const h8*>(xs + arow * kQ8RowBytes + 2 * (512 * wave + 32 * st + 8 * h));
    __builtin_amdgcn_sched_barrier(0);

    // Two accumulators alternate along a chain so that consecutive matrix-core
    // products do not wait for each other; a chain's first two steps start
    // from the constant zero.
    f32x4 c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
    const f32x4 zero4 = c0;
#pragma unroll
    for (int i = 0; i < kQ8Tiles; ++i) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int st = 2 * i + s;
        const uint32_t d0 = wv[i][2 * s], d1 = wv[i][2 * s + 1];
        const u32x4 bw = {q8_byte_pair<0>(d0), q8_byte_pair<1>(d0), q8_byte_pair<0>(d1),
                          q8_byte_pair<1>(d1)};
        const h8 b = __builtin_bit_cast(h8, bw);
        const int pos = st % CL;
        if (pos == 0)
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], b, zero4, 0, 0, 0);
        else if (pos == 1)
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], b, zero4, 0, 0, 0);
        else if (pos % 2 == 0)
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], b, c0, 0, 0, 0);
        else
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st], b, c1, 0, 0, 0);
        if (pos == CL - 1) {
          const int c = st / CL;
          const float* off = &cs[wave * NC + c][4 * h];
#pragma unroll
          for (int r = 0; r < RR; ++r) {
            const float v = CL == 1 ? c0[r] : c0[r] + c1[r];
            tot[r] = __builtin_fmaf(v + off[r], sc[c], tot[r]);
          }
        }
      }
    }
  }

  // The 8 waves' totals, added in wave order.
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    const int row = 4 * h + r;
    if (row < MT) red[wave][row][j] = tot[r];
  }
  __syncthreads();
  if (t < MT * 16) {
    const int row = t >> 4, col = t & 15;
    float s = red[0][row][col];
#pragma unroll
    for (int w = 1; w < kQ8Waves; ++w) s += red[w][row][col];
    if (row < M) Y[(size_t)row * N + 16 * panel + col] = (_Float16)(s * kTwo24);
  }
}

hipError_t launch_q8_prepack(const int8_t* W, void* packed, int K, int N, hipStream_t s) {
  const size_t total = (size_t)(N / 16) * q8_tiles_per_panel(K) * 64;
  hipLaunchKernelGGL(q8_prepack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, W, reinterpret_cast<uint8_t*>(packed), K, N);
  return hipGetLastError();
}

hipError_t launch_q8_unpack(const void* packed, int8_t* codes, int K, int N, hipStream_t s) {
  const size_t total = (size_t)(N / 16) * q8_tiles_per_panel(K) * 64;
  hipLaunchKernelGGL(q8_unpack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint8_t*>(packed), codes, K, N);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_q8_rows(const void* X, const void* packed, const float* scales, void* Y,
                                 int M, int K, int N, int G, hipStream_t s) {
  const int KT = q8_tiles_per_panel(K);
  const bool pow2 = (G & (G - 1)) == 0;
  const int CL = !pow2 ? 1 : G >= 512 ? 16 : G / 32;
  const dim3 grid(N / 16), block(kQ8Threads);
  const _Float16* x = reinterpret_cast<const _Float16*>(X);
  const uint8_t* w = reinterpret_cast<const uint8_t*>(packed);
  _Float16* y = reinterpret_cast<_Float16*>(Y);
  switch (CL) {
    case 16: hipLaunchKernelGGL((q8_mfma_kernel<MT, 16>), grid, block, 0, s, x, w, scales, y, M, K, N, G, KT); break;
    case 8: hipLaunchKernelGGL((q8_mfma_kernel<MT, 8>), grid, block, 0, s, x, w, scales, y, M, K, N, G, KT); break;
    case 4: hipLaunchKernelGGL((q8_mfma_kernel<MT, 4>), grid, block, 0, s, x, w, scales, y, M, K, N, G, KT); break;
    case 2: hipLaunchKernelGGL((q8_mfma_kernel<MT, 2>), grid, block, 0, s, x, w, scales, y, M, K, N, G, KT); break;
    default: hipLaunchKernelGGL((q8_mfma_kernel<MT, 1>), grid, block, 0, s, x, w, scales, y, M, K, N, G, KT); break;
  }
  return hipGetLastError();
}

size_t q8_group_workspace_bytes(int M, int K, int N) {
  return M >= kQ8GemmMinRows ? q8_gemm_workspace_bytes(M, K, N) : 0;
}

hipError_t launch_q8_group(const void* X, const void* packed, const float* scales, void* Y,
                           void* ws, int M, int K, int N, int G, hipStream_t s) {
  if (M >= kQ8GemmMinRows && q8_gemm_supported(M, K, N, G))
    return launch_q8_gemm(X, packed, scales, Y, ws, M, K, N, G, s);
  // Up to 16 rows of X per launch over the same weight.
  for (int m0 = 0; m0 < M; m0 += kQ8PassRows) {
    const int mc = (M - m0) < kQ8PassRows ? (M - m0) : kQ8PassRows;
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)m0 * K * 2;
    void* Yc = reinterpret_cast<char*>(Y) + (size_t)m0 * N * 2;
    hipError_t e;
    if (mc == 1)
      e = launch_q8_rows<1>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else if (mc == 2)
      e = launch_q8_rows<2>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else if (mc <= 4)
      e = launch_q8_rows<4>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else if (mc <= 8)
      e = launch_q8_rows<8>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else
      e = launch_q8_rows<16>(Xc, packed, scales, Yc, mc, K, N, G, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
