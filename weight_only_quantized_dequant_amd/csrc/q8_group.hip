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
// The product at one or two rows of X.  A wave owns one column pair over all
// of K, so no partial sum ever leaves the wave: at step i lane l takes piece
// 64 i + l of its pair (the wave reads 1 KB of contiguous memory per step),
// and one cross-lane reduction at the end gives the two outputs.  Eight waves
// (a 16-column panel) share the activations, staged once per 4096 rows in LDS.
//
// The product at 3 .. 16 rows (q8_mfma_kernel) runs on the matrix cores,
// v_mfma_f32_16x16x32_f16, from the same packed weight: the 8 waves of a
// panel split K, each load instruction of a wave brings 128 contiguous bytes
// of each of the panel's 8 pairs, and a wave-private LDS copy turns them into
// the operand order (16 columns x 32 rows per step).  At 17 .. 32 rows
// (q8_mfma32_kernel) each step takes two 16-row tiles of X, staged per
// 2048-row chunk.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// 512 threads (8 wave64s, two per SIMD): while one wave of a SIMD converts
// its codes the other's loads are still landing.
constexpr int kQ8Threads = 512;
constexpr int kQ8Steps = 8;                    // pieces per lane per chunk
constexpr int kQ8Chunk = 64 * kQ8Steps * 8;    // rows of K per chunk: 4096
// From this many rows of X on, the product runs as a tiled matrix-core GEMM
// (q8_gemm.hip) instead of one streaming pass over the weight per 32 rows.
constexpr int kQ8GemmMinRows = 33;
constexpr int kQ8PassRows = 32;

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

// x from lane (l - R) mod 16 of this lane's 16-lane row (DPP row_ror:R).
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

// ONE (one row of X, FOLD, K exactly one 4096-row chunk): straight-line code
// with no range selects, and the activation and scale requests pinned ahead
// of the weight stream (the compiler otherwise hoists the sums of x above the
// weight loads, and each wave then waits for its activations before it asks
// for any weights).
template <int MT, bool FOLD, bool ONE = false>
__global__ __launch_bounds__(kQ8Threads) void q8_pair_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const float* __restrict__ scales, _Float16* __restrict__ Y, int M, int K, int N, int G,
    int gsh, int ngroups) {
  static_assert(!ONE || (MT == 1 && FOLD), "the single-chunk form is for one row");
  // The host launches with K >= 32: the first chunk is unconditional, so
  // the kernel arguments can be requested in one batch.
  __builtin_assume(K > 0);
  if constexpr (!ONE) asm volatile("" ::"s"(X), "s"(Wp), "s"(scales));
  if constexpr (ONE) {
    M = 1;
    K = kQ8Chunk;
  }
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
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, ngroups * N * 4);  // ngroups = K / G

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
    for (int m = 0; m < MT; ++m) {
      if constexpr (ONE)  // one row, one chunk, 8 t < 4096: always in range
        xg[m] = __builtin_amdgcn_raw_buffer_load_b128(xr, 16 * t, 0, 0);
      else
        xg[m] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, (m < M && r0 + 8 * t < K) ? (m * K + r0 + 8 * t) * 2 : kOutOfRange, 0, 0);
    }
    if constexpr (ONE) {  // the activation load goes out first (IR and machine order)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
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
    if constexpr (ONE) __builtin_amdgcn_sched_barrier(0);
    u32x4 w[kQ8Steps];
#pragma unroll
    for (int i = 0; i < kQ8Steps; ++i) {
      const int b = b0 + 64 * i + lane;
      w[i] = buffer_stream(wr, b < KB ? (q * KB + b) * 16 : kOutOfRange);
    }
    wait_vmcnt<kQ8Steps + NS>();  // the activations have landed
    if constexpr (ONE) asm volatile("" : "+v"(xg[0])::"memory");
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

// ---------------------------------------------------------------------------
// The product at 3 .. 16 rows of X, on the matrix cores.
//
// A workgroup of 8 waves owns a panel (8 column pairs, 16 columns); of every
// 4096-row chunk wave w takes rows 512 w .. 512 w + 511.  Its load i brings
// rows 64 i .. 64 i + 63 of that range for all 8 pairs: lane l the piece
// 8 i + l % 8 of pair l / 8, so each instruction reads 8 whole 128-byte
// runs.  The wave writes the loaded KB into its own LDS slot and reads it
// back in the operand order of v_mfma_f32_16x16x32_f16: for step 2 i + s,
// lane l (column l % 16, rows 8 (l / 16) .. + 7 of the step) takes the piece
// 4 s + l / 16 of pair (l % 16) / 2, and one v_perm_b32 per word keeps its
// column's two code bytes as an fp16 pair (the subnormals u 2^-24).  X
// (up to 16 rows) is the A operand, read from the LDS copy of the chunk (row
// l % 16 of the operand; rows past M are zero).  The offset 128 comes out per
// chain of steps inside one group: the staging threads form
// -128 2^-24 sum(x) over each chain's rows once per workgroup, and a chain's
// sums take it before the scale: total += (chain sums + offset) * scale, in
// fp32, in units of 2^-24.  The 8 waves' totals are added in a fixed order.
// ---------------------------------------------------------------------------
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// LDS row of X: a chunk of fp16 plus 16 bytes, so that the 16 rows an
// operand read takes start on different banks.
constexpr int kQ8RowBytes = 2 * kQ8Chunk + 16;
constexpr int kQ8Waves = kQ8Threads / 64;

// s_waitcnt vmcnt(left) for a count known once the loop around it is
// unrolled.
__device__ __forceinline__ void wait_vmcnt_dyn(int left) {
  switch (left) {
    case 7: wait_vmcnt<7>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 1: wait_vmcnt<1>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

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
    int gsh, int ngroups) {
  // The host launches with K >= 32: the first chunk is unconditional, so
  // the kernel arguments can be requested in one batch.
  __builtin_assume(K > 0);
  asm volatile("" ::"s"(scales));
  constexpr int NSTEP = 16;                    // 32-row steps per wave per chunk
  constexpr int NC = NSTEP / CL;               // chains per wave per chunk
  constexpr int NG = kQ8Chunk / (32 * CL);     // chains per chunk
  constexpr int RR = MT < 4 ? MT : 4;          // accumulator rows that can hold rows of X
  static_assert(CL == 1 || CL == 2 || CL == 4 || CL == 8 || CL == 16, "chain length");
  static_assert(kQ8Waves == 8 && kQ8Chunk == 512 * kQ8Waves, "a wave takes 512 rows of a chunk");
  __shared__ __attribute__((aligned(16))) unsigned char xs[MT * kQ8RowBytes];  // the chunk of X
  __shared__ float cs[NG][16];  // [chain][row of X]: -128 2^-24 sum of x over the chain's rows
  // Per wave: the slots of the operand reorder (its totals at the end).  At
  // 8 rows of X (DL) the loads go straight to LDS, one 1 KB slot each (the
  // compiler then waits for all eight before the first read; measured
  // 6.17 -> 5.98 us at M = 8, but 5.19 -> 5.36 at M = 4); otherwise they land
  // in registers and pass through two slots (at 16 rows the LDS holds no
  // eight).
  constexpr bool DL = MT == 8;
  constexpr int SLOTS = DL ? 8 : 2;
  __shared__ __attribute__((aligned(1024))) unsigned char tr[kQ8Waves][SLOTS * 1024];

  const int t = threadIdx.x, lane = t & 63, h = lane >> 4, j = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Workgroups b and b + 8 run on the same XCD (dispatch is round-robin over
  // the 8 XCDs).  When the panel count allows, they take neighbouring panels,
  // which share the 128-byte lines of the fp32 scale rows.
  const int bid = blockIdx.x;
  const int panel = (gridDim.x % 16 == 0) ? (bid & ~15) + 2 * (bid & 7) + ((bid >> 3) & 1) : bid;
  const int KB = K / 8;  // pieces per pair

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, K * N);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, ngroups * N * 4);  // ngroups = K / G

  // tot[r]: row 4 (l / 16) + r of X, column 16 panel + l % 16, units of 2^-24.
  float tot[RR];
#pragma unroll
  for (int r = 0; r < RR; ++r) tot[r] = 0.0f;
  const int arow = j < MT ? j : 0;                           // row of X in this lane's A operand
  const int lpair = 8 * panel + (lane >> 3);                 // pair this lane loads
  const uint32_t sel = (j & 1) ? 0x0c030c02u : 0x0c010c00u;  // its operand column in a piece
  unsigned char* mytr = &tr[wave][0];

  for (int r0 = 0; r0 < K; r0 += kQ8Chunk) {
    // Activations first (rows r0 + 8t .. + 7; zero past K and for m >= M),
    // then the scales, then the weight, so waiting for the activations
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
      const int g = gsh >= 0 ? row >> gsh : row / G;  // gsh = log2 G, or -1
      sc[c] = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
          sr, row < K ? (g * N + 16 * panel + j) * 4 : kOutOfRange, 0, 0));
    }
    const int b0 = (r0 + 512 * wave) / 8;
    u32x4 wv[DL ? 1 : 8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int b = b0 + 8 * i + (lane & 7);
      const int off = b < KB ? (lpair * KB + b) * 16 : kOutOfRange;
      if constexpr (DL)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            wr, (__attribute__((address_space(3))) void*)(mytr + 1024 * i), 16, off, 0, 0, 2);
      else
        wv[i] = buffer_stream(wr, off);
    }
    wait_vmcnt<NC + 8>();       // the activations have landed
    if (r0 > 0) lds_barrier();  // every wave is done with the previous chunk
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
      ps += q8_dpp<0xB1>(ps);                          // quad_perm 1 0 3 2
      ps += q8_dpp<0x4E>(ps);                          // quad_perm 2 3 0 1
      if constexpr (CL >= 2) ps += q8_dpp<0x12C>(ps);  // row_ror:12, lane l + 4
      if constexpr (CL >= 4) ps += q8_dpp<0x128>(ps);  // row_ror:8
      if constexpr (CL >= 8) ps += __shfl_xor(ps, 16);
      if constexpr (CL >= 16) ps += __shfl_xor(ps, 32);
      if ((t & (4 * CL - 1)) == 0) cs[t / (4 * CL)][m] = ps;
    }
    lds_barrier();

    // Every step's A operand before any weight is waited for (the
    // scheduling barrier keeps the compiler from sinking the reads).
    h8 av[NSTEP];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
      av[st] = *reinterpret_cast<const h8*>(xs + arow * kQ8RowBytes + 2 * (512 * wave + 32 * st + 8 * h));
    __builtin_amdgcn_sched_barrier(0);

    // Two accumulators alternate along a chain so that consecutive matrix-core
    // products do not wait for each other; a chain's first two steps start
    // from the constant zero.
    f32x4 c0 = {0.0f, 0.0f, 0.0f, 0.0f}, c1 = c0;
    const f32x4 zero4 = c0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // The loaded KB into this wave's slot.  The LDS executes one wave's
      // accesses in issue order, so the reads below see every lane's write
      // (and a slot is rewritten only after its reads) without a wait.
      unsigned char* slot = mytr + 1024 * (DL ? i : (i & 1));
      if constexpr (DL) {
        wait_vmcnt_dyn(7 - i);  // load i has reached LDS (the later loads may not)
      } else {
        *reinterpret_cast<u32x4*>(slot + 16 * lane) = wv[i];
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int st = 2 * i + s;
        const u32x4 pc = *reinterpret_cast<const u32x4*>(slot + 16 * (8 * (j >> 1) + 4 * s + h));
        const u32x4 bw = {__builtin_amdgcn_perm(0u, pc[0], sel), __builtin_amdgcn_perm(0u, pc[1], sel),
                          __builtin_amdgcn_perm(0u, pc[2], sel), __builtin_amdgcn_perm(0u, pc[3], sel)};
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
      asm volatile("" ::: "memory");
    }
  }

  // The 8 waves' totals (each in its own slot), added as a fixed-order
  // pairwise tree ((w0 + w1) + (w2 + w3)) + ((w4 + w5) + (w6 + w7)).
  float* red = reinterpret_cast<float*>(mytr);  // [MT][16]
#pragma unroll
  for (int r = 0; r < RR; ++r) {
    const int row = 4 * h + r;
    if (row < MT) red[row * 16 + j] = tot[r];
  }
  __syncthreads();
  if (t < MT * 16) {
    const int row = t >> 4, col = t & 15;
    float v[kQ8Waves];
#pragma unroll
    for (int w = 0; w < kQ8Waves; ++w) v[w] = reinterpret_cast<const float*>(&tr[w][0])[row * 16 + col];
    const float s = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    if (row < M) Y[(size_t)row * N + 16 * panel + col] = (_Float16)(s * kTwo24);
  }
}

// ---------------------------------------------------------------------------
// The product at 17 .. 32 rows of X: q8_mfma_kernel's scheme with two 16-row
// tiles of X per step (two matrix-core products per weight operand) and X
// staged per 2048-row chunk (32 rows of a 4096-row chunk do not fit the LDS):
// of every chunk wave w takes rows 256 w .. 256 w + 255, four 1 KB loads.
// Thread t stages piece t % 256 (8 rows of K) of the rows t / 256 + 2 i of X.
// CL: 32-row steps per chain (one scale), at most the wave's 8 steps of a
// chunk: G / 32 for groups of 32 .. 256 rows, 8 for larger powers of two, 1
// for other group sizes.
// ---------------------------------------------------------------------------
template <int CL>
__global__ __launch_bounds__(kQ8Threads) void q8_mfma32_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const float* __restrict__ scales, _Float16* __restrict__ Y, int M, int K, int N, int G,
    int gsh, int ngroups) {
  constexpr int MT = 32, CH = 2048;
  constexpr int NL = CH / (64 * kQ8Waves);    // 1 KB loads per wave per chunk: 4
  constexpr int NSTEP = 2 * NL;               // 32-row steps per wave per chunk: 8
  constexpr int WR = CH / kQ8Waves;           // rows per wave per chunk: 256
  constexpr int NC = NSTEP / CL;              // chains per wave per chunk
  constexpr int NG = CH / (32 * CL);          // chains per chunk
  constexpr int XRB = 2 * CH + 16;            // LDS bytes per row of X (bank spread)
  constexpr int PPR = CH / 8;                 // 16-byte pieces per row of a chunk: 256
  constexpr int XPT = MT * PPR / kQ8Threads;  // pieces of X per thread per chunk: 16
  static_assert(CL == 1 || CL == 2 || CL == 4 || CL == 8, "chain length");
  static_assert(kQ8Threads == 2 * PPR, "two row parities of 256 pieces");
  __shared__ __attribute__((aligned(16))) unsigned char xs[MT * XRB];  // the chunk of X
  __shared__ float cs[NG][MT];  // [chain][row of X]: -128 2^-24 sum of x over the chain's rows
  __shared__ __attribute__((aligned(1024))) unsigned char tr[kQ8Waves][2 * 1024];

  const int t = threadIdx.x, lane = t & 63, h = lane >> 4, j = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int bid = blockIdx.x;
  const int panel = (gridDim.x % 16 == 0) ? (bid & ~15) + 2 * (bid & 7) + ((bid >> 3) & 1) : bid;
  const int KB = K / 8;  // pieces per pair

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, K * N);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, ngroups * N * 4);  // ngroups = K / G

  // tot[tt][r]: row 16 tt + 4 (l / 16) + r of X, column 16 panel + l % 16, units of 2^-24.
  float tot[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) tot[tt][r] = 0.0f;
  const int lpair = 8 * panel + (lane >> 3);                 // pair this lane loads
  const uint32_t sel = (j & 1) ? 0x0c030c02u : 0x0c010c00u;  // its operand column in a piece
  unsigned char* mytr = &tr[wave][0];
  const int xp = t & (PPR - 1), xq = t / PPR;  // staged piece and row parity

  // Chunk c + 1's activations, scales and weight are requested before chunk
  // c's products (into registers), so only the first chunk waits for a full
  // round trip; the next chunk's X is staged once every wave is done with
  // the current one.
  u32x4 xg[XPT];
  float sc[NC], scn[NC];
  u32x4 wv[NL], wn[NL];
  auto issue = [&](int r0, u32x4 (&xgr)[XPT], float (&scr)[NC], u32x4 (&wvr)[NL]) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int m = xq + 2 * i;
      xgr[i] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, (r0 < K && m < M && r0 + 8 * xp < K) ? (m * K + r0 + 8 * xp) * 2 : kOutOfRange, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int row = r0 + WR * wave + 32 * CL * c;
      const int g = gsh >= 0 ? row >> gsh : row / G;  // gsh = log2 G, or -1
      scr[c] = as_f32(__builtin_amdgcn_raw_buffer_load_b32(
          sr, row < K ? (g * N + 16 * panel + j) * 4 : kOutOfRange, 0, 0));
    }
    const int b0 = (r0 + WR * wave) / 8;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int b = b0 + 8 * i + (lane & 7);
      wvr[i] = buffer_stream(wr, (r0 < K && b < KB) ? (lpair * KB + b) * 16 : kOutOfRange);
    }
  };
  issue(0, xg, sc, wv);

  for (int r0 = 0; r0 < K; r0 += CH) {
    wait_vmcnt<NC + NL>();      // this chunk's activations have landed
    if (r0 > 0) lds_barrier();  // every wave is done with the previous chunk
    // Stage X; the chain sums: piece xp lies in chain xp / (4 CL), whose 4 CL
    // threads are consecutive lanes (fixed-order DPP sums).
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int m = xq + 2 * i;
      *reinterpret_cast<u32x4*>(xs + m * XRB + 16 * xp) = xg[i];
      const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
      float ps = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) ps = dot2(as_h2(xg[i][d]), ones, ps);
      ps *= -128.0f / kTwo24;
      ps += q8_dpp<0xB1>(ps);                          // quad_perm 1 0 3 2
      ps += q8_dpp<0x4E>(ps);                          // quad_perm 2 3 0 1
      if constexpr (CL >= 2) ps += q8_dpp<0x12C>(ps);  // row_ror:12, lane l + 4
      if constexpr (CL >= 4) ps += q8_dpp<0x128>(ps);  // row_ror:8
      if constexpr (CL >= 8) ps += __shfl_xor(ps, 16);
      if ((xp & (4 * CL - 1)) == 0) cs[xp / (4 * CL)][m] = ps;
    }
    lds_barrier();

    // Every step's two A operands, then the next chunk's loads.
    h8 av[NSTEP][2];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = 16 * tt + j < M ? 16 * tt + j : 0;
        av[st][tt] = *reinterpret_cast<const h8*>(xs + row * XRB + 2 * (WR * wave + 32 * st + 8 * h));
      }
    issue(r0 + CH, xg, scn, wn);  // past the last chunk: out of range, no request
    __builtin_amdgcn_sched_barrier(0);

    // Two accumulators per tile alternate along a chain; a chain's first two
    // steps start from the constant zero.
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    f32x4 c0[2] = {zero4, zero4}, c1[2] = {zero4, zero4};
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      // The loaded KB into this wave's slot (a wave's LDS accesses run in
      // issue order: no wait between the write and the reads).
      unsigned char* slot = mytr + 1024 * (i & 1);
      *reinterpret_cast<u32x4*>(slot + 16 * lane) = wv[i];
      asm volatile("" ::: "memory");
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int st = 2 * i + s;
        const u32x4 pc = *reinterpret_cast<const u32x4*>(slot + 16 * (8 * (j >> 1) + 4 * s + h));
        const u32x4 bw = {__builtin_amdgcn_perm(0u, pc[0], sel), __builtin_amdgcn_perm(0u, pc[1], sel),
                          __builtin_amdgcn_perm(0u, pc[2], sel), __builtin_amdgcn_perm(0u, pc[3], sel)};
        const h8 b = __builtin_bit_cast(h8, bw);
        const int pos = st % CL;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          if (pos == 0)
            c0[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st][tt], b, zero4, 0, 0, 0);
          else if (pos == 1)
            c1[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st][tt], b, zero4, 0, 0, 0);
          else if (pos % 2 == 0)
            c0[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st][tt], b, c0[tt], 0, 0, 0);
          else
            c1[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[st][tt], b, c1[tt], 0, 0, 0);
        }
        if (pos == CL - 1) {
          const int c = st / CL;
          const float* off = &cs[wave * NC + c][0];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = CL == 1 ? c0[tt][r] : c0[tt][r] + c1[tt][r];
              tot[tt][r] = __builtin_fmaf(v + off[16 * tt + 4 * h + r], sc[c], tot[tt][r]);
            }
        }
      }
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) sc[c] = scn[c];
#pragma unroll
    for (int i = 0; i < NL; ++i) wv[i] = wn[i];
  }

  // The 8 waves' totals (each in its own 2 KB slot), added as a fixed-order
  // pairwise tree ((w0 + w1) + (w2 + w3)) + ((w4 + w5) + (w6 + w7)).
  float* red = reinterpret_cast<float*>(mytr);  // [32][16]
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(16 * tt + 4 * h + r) * 16 + j] = tot[tt][r];
  __syncthreads();
  {
    const int row = t >> 4, col = t & 15;  // 512 threads: the 32 x 16 outputs
    float v[kQ8Waves];
#pragma unroll
    for (int w = 0; w < kQ8Waves; ++w) v[w] = reinterpret_cast<const float*>(&tr[w][0])[row * 16 + col];
    const float s = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    if (row < M) Y[(size_t)row * N + 16 * panel + col] = (_Float16)(s * kTwo24);
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
  if constexpr (MT == 1 && FOLD) {
    if (K == kQ8Chunk) {
      hipLaunchKernelGGL((q8_pair_kernel<1, true, true>), dim3(N / 16), dim3(kQ8Threads), 0, s,
                         reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                         scales, reinterpret_cast<_Float16*>(Y), M, K, N, G, gsh, K / G);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((q8_pair_kernel<MT, FOLD>), dim3(N / 16), dim3(kQ8Threads), 0, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                     scales, reinterpret_cast<_Float16*>(Y), M, K, N, G, gsh, K / G);
  return hipGetLastError();
}

template <int MT>
static hipError_t launch_q8_rows(const void* X, const void* packed, const float* scales, void* Y,
                                 int M, int K, int N, int G, hipStream_t s) {
  const bool pow2 = (G & (G - 1)) == 0;
  const int CL = !pow2 ? 1 : G >= 512 ? 16 : G / 32;
  int gsh = -1;
  if (pow2)
    for (gsh = 0; (1 << gsh) < G; ++gsh) {
    }
  const dim3 grid(N / 16), block(kQ8Threads);
  const _Float16* x = reinterpret_cast<const _Float16*>(X);
  const uint8_t* w = reinterpret_cast<const uint8_t*>(packed);
  _Float16* y = reinterpret_cast<_Float16*>(Y);
  switch (CL) {
    case 16: hipLaunchKernelGGL((q8_mfma_kernel<MT, 16>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
    case 8: hipLaunchKernelGGL((q8_mfma_kernel<MT, 8>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
    case 4: hipLaunchKernelGGL((q8_mfma_kernel<MT, 4>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
    case 2: hipLaunchKernelGGL((q8_mfma_kernel<MT, 2>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
    default: hipLaunchKernelGGL((q8_mfma_kernel<MT, 1>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
  }
  return hipGetLastError();
}

// 17 .. 32 rows: one pass of q8_mfma32_kernel.
static hipError_t launch_q8_rows32(const void* X, const void* packed, const float* scales, void* Y,
                                   int M, int K, int N, int G, hipStream_t s) {
  const bool pow2 = (G & (G - 1)) == 0;
  const int CL = !pow2 ? 1 : G >= 256 ? 8 : G / 32;
  int gsh = -1;
  if (pow2)
    for (gsh = 0; (1 << gsh) < G; ++gsh) {
    }
  const dim3 grid(N / 16), block(kQ8Threads);
  const _Float16* x = reinterpret_cast<const _Float16*>(X);
  const uint8_t* w = reinterpret_cast<const uint8_t*>(packed);
  _Float16* y = reinterpret_cast<_Float16*>(Y);
  switch (CL) {
    case 8: hipLaunchKernelGGL((q8_mfma32_kernel<8>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
    case 4: hipLaunchKernelGGL((q8_mfma32_kernel<4>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
    case 2: hipLaunchKernelGGL((q8_mfma32_kernel<2>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
    default: hipLaunchKernelGGL((q8_mfma32_kernel<1>), grid, block, 0, s, x, w, scales, y, M, K, N, G, gsh, K / G); break;
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
  // Up to 32 rows of X per launch over the same weight: one or two rows on
  // the v_dot2 pair kernel, 3 .. 32 on the matrix cores.
  for (int m0 = 0; m0 < M; m0 += kQ8PassRows) {
    const int mc = (M - m0) < kQ8PassRows ? (M - m0) : kQ8PassRows;
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
    else if (mc <= 4)
      e = launch_q8_rows<4>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else if (mc <= 8)
      e = launch_q8_rows<8>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else if (mc <= 16)
      e = launch_q8_rows<16>(Xc, packed, scales, Yc, mc, K, N, G, s);
    else
      e = launch_q8_rows32(Xc, packed, scales, Yc, mc, K, N, G, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
