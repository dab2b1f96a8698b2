// 4-bit symmetric group-wise weight-only GEMM (small M), with act-order.
//
//   Y[m, n] = sum_g scale[g, n] * sum_{rows i of group g} X[m, perm[i]] * q'[i, n]
//
// Codes are 8 per int32 along K, stored as u = q + 8 ("Quantization CUDA",
// tom-jerr.github.io, sections "Int4 Weight Only Quantization" and "Weight
// Store"; "量化粒度": group-wise scales, groups of 128 along K).  With
// act-order ("GPTQ算法解析", intelliparadigm.com, section 4.1: act_order) a
// row's group g_idx[k] is not monotone in k.  The weight is re-laid out once,
// offline (wq_prepack_q4), the same idea as the offline re-layout of "Marlin
// 格式" on the "Quantization CUDA" page: rows are put in group order (perm),
// then into the operand order of the matrix cores; the inverse permutation
// travels with the packed weight as a uint16 row table.  At run time each
// workgroup scatters X into LDS through that table (coalesced reads, LDS
// writes), so the rows the cores combine are one group at a time.
//
// The products run on v_mfma_f32_16x16x32_f16 for every M (rows of X past M
// are zero lanes of the operand).  A code u (0..15) enters the cores as the
// fp16 subnormal with mantissa u, i.e. exactly u * 2^-24, so each product
// x * u * 2^-24 is exact in the fp32 accumulator.  Per group g the tile
//   C = sum_k x[m, k] u[k, n] 2^-24   and the group sum  S = sum_k x[m, k]
// give the group's share  scale[g, n] * (C - 8 * 2^-24 * S)  of Y / 2^24:
// the (u - 8) offset is applied once per group, not per code.  S depends on
// X only, so each workgroup computes it once per (row, group) from the X it
// staged in LDS and every panel reuses it.
//
// Layout.  Panels of 16 columns; a panel's rows (group order) are cut into
// blocks of 128, zero-padded to a whole block.  Block (panel p, block b) is
// 1 KB: lane l owns 16 bytes = 4 words, word j holding the 8 codes of column
// 16 p + l % 16, rows 128 b + 32 j + 8 (l / 16) .. +7, row +e in nibble e —
// the B operand of MFMA step j of the block, one 1 KB load per wave.
//
// 2-bit codes (named on "GPTQ CUDA kernel walkthrough", yelogs.com, as a
// lower bit width to support) run through the same kernel in the asymmetric
// form: blocks of 256 rows, word j of a lane holding the 16 codes of steps
// 2j and 2j + 1 (rows 256 b + 64 j + 8 (l / 16) + e and 32 rows further),
// placed so that (w >> 2i) & 0x00030003 is the operand pair i: pairs 0..3
// are step 2j's rows (e, e + 4), pairs 4..7 step 2j + 1's.
#include "q4_layout.hpp"
#include "wq_internal.h"

namespace wq {

constexpr int kQ4Ring = 4;     // blocks in flight per wave
constexpr int kQ4MaxRun = 8;   // panels a workgroup walks at most
constexpr int kQ4Threads = 512;             // 8 waves: two per SIMD
constexpr int kQ4Waves = kQ4Threads / 64;
// Padding (halves) after each LDS row of X: 4 octets, so the 16-byte operand
// reads of rows m and octets o fall on banks 4 m + o (mod 16 groups).
constexpr int kQ4RowPad = 32;

// PanelPlan for the 4-bit layout: P = 16, npanels = ceil(N / 16),
// u = blocks per panel = ceil(K / 128); cpp, nsa and bw are unused.  The
// packed weight is the blocks, then the row table: K uint16, entry k = the
// group-order row of original row k (the inverse of perm), padded to 16 B.
// The 4-bit weight then holds the forward table too (q4_fwd_table_offset):
// u * 128 uint16, entry i = the original row of group-order row i (perm[i]),
// 0xFFFF for the padding rows K .. u * 128 - 1.
static size_t q4_block_bytes(const PanelPlan& p) { return (size_t)p.npanels * p.u * 1024; }
static size_t q4_inv_table_bytes(int K) { return ((size_t)K * 2 + 15) / 16 * 16; }
static PanelPlan plan_blocks(int K, int N, int rows, bool fwd) {
  PanelPlan p{};
  p.P = kQ4Panel;
  p.cpp = 0;
  p.npanels = (N + kQ4Panel - 1) / kQ4Panel;
  p.u = (K + rows - 1) / rows;
  p.nsa = 0;
  p.bw = 0;
  p.packed_bytes = q4_block_bytes(p) + q4_inv_table_bytes(K) + (fwd ? (size_t)p.u * rows * 2 : 0);
  return p;
}
PanelPlan plan_q4(int K, int N, int G) {
  (void)G;
  return plan_blocks(K, N, block_rows<4>(), true);
}
size_t q4_fwd_table_offset(int K, int N) {
  return q4_block_bytes(plan_blocks(K, N, block_rows<4>(), true)) + q4_inv_table_bytes(K);
}
// 2-bit: the same structure with 256-row blocks (no forward table).
PanelPlan plan_q2(int K, int N, int G) {
  (void)G;
  return plan_blocks(K, N, block_rows<2>(), false);
}

// Rows of X staged per launch: the LDS copies of X (MT rows of the padded
// block rows plus padding) stay <= 96 KB.
static int max_mt(int K, int rows) {
  const size_t kb = (size_t)(K + rows - 1) / rows * rows + kQ4RowPad;
  int mt = 8;
  while (mt > 1 && (size_t)mt * kb * 2 > 98304) mt /= 2;
  return mt;
}

// Code pairs of one word as fp16 subnormals: (e, e + 4) for e = 0..3, i.e.
// the 8 rows in the order 0 4 1 5 2 6 3 7 — the order X takes in LDS.
__device__ __forceinline__ void q4_mfma_pairs(uint32_t w, h2 out[4]) {
  out[0] = as_h2(w & 0x000F000Fu);
  out[1] = as_h2((w >> 4) & 0x000F000Fu);
  out[2] = as_h2((w >> 8) & 0x000F000Fu);
  out[3] = as_h2((w >> 12) & 0x000F000Fu);
}
// 2-bit: the operand of step 2j + H of word j: pairs 4H .. 4H + 3, i.e.
// (w >> 2i) & 0x00030003, each half an exact subnormal u * 2^-24.
template <int H>
__device__ __forceinline__ void q2_mfma_pairs(uint32_t w, h2 out[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = as_h2((w >> (2 * (4 * H + i))) & 0x00030003u);
}
template <int H>
__device__ __forceinline__ u32x4 q2_mfma_operand(uint32_t w) {
  constexpr int b = 8 * H;
  return u32x4{(w >> b) & 0x00030003u, (w >> (b + 2)) & 0x00030003u,
               (w >> (b + 4)) & 0x00030003u, (w >> (b + 6)) & 0x00030003u};
}
// Code position (0..15) of row e of step 2j + H inside word j.
__host__ __device__ constexpr int q2_pos(int h, int e) { return e < 4 ? e + 4 * h : e + 4 + 4 * h; }


// ---------------------------------------------------------------------------
// Offline re-layout: one thread per (panel, block, lane) 16-byte piece.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q4_prepack_kernel(const uint32_t* __restrict__ qw,
                                                              const int* __restrict__ perm,
                                                              uint32_t* __restrict__ out,
                                                              uint16_t* __restrict__ table,
                                                              uint16_t* __restrict__ fwd, int K,
                                                              int N, int nb, int npanels) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  // Row tables: table[perm[i]] = i and fwd[i] = perm[i].  Entries of perm
  // outside 0..K-1 (perm not a permutation: a broken precondition) are
  // skipped in table and stored as 0xFFFF (no row) in fwd, never used as an
  // address.
  for (size_t i = idx; i < (size_t)nb * kQ4Block; i += (size_t)gridDim.x * kThreads) {
    const int k = i < (size_t)K ? (perm ? perm[i] : (int)i) : -1;
    const bool ok = k >= 0 && k < K;
    if (ok) table[k] = (uint16_t)i;
    fwd[i] = ok ? (uint16_t)k : (uint16_t)0xFFFFu;
  }
  if (idx >= (size_t)npanels * nb * 64) return;
  const int l = (int)(idx % 64);
  const size_t pb = idx / 64;
  const int b = (int)(pb % nb), panel = (int)(pb / nb);
  const int n = panel * kQ4Panel + l % 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i0 = kQ4Block * b + 32 * j + 8 * (l / 16);
    uint32_t word = 0;  // padding rows and columns: u = 0, met by x = 0 or dropped
    if (n < N) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = i0 + e;
        if (i >= K) break;
        const int src = perm ? perm[i] : i;
        if (src < 0 || src >= K) continue;
        const uint32_t sw = qw[(size_t)(src >> 3) * N + n];
        word |= ((sw >> (4 * (src & 7))) & 15u) << (4 * e);
      }
    }
    out[idx * 4 + j] = word;
  }
}

// 2-bit: qw [K/16, N], row 16 r + j in bits 2j, 2j + 1 of word r.  Piece
// (panel, block b, lane l), word j: the rows of steps 2j + h (h = 0, 1),
// 256 b + 64 j + 32 h + 8 (l / 16) + e, at code position q2_pos(h, e).
__global__ __launch_bounds__(kThreads) void q2_prepack_kernel(const uint32_t* __restrict__ qw,
                                                              const int* __restrict__ perm,
                                                              uint32_t* __restrict__ out,
                                                              uint16_t* __restrict__ table, int K,
                                                              int N, int nb, int npanels) {
  constexpr int BR = block_rows<2>();
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (size_t i = idx; i < (size_t)K; i += (size_t)gridDim.x * kThreads) {
    const int k = perm ? perm[i] : (int)i;
    if (k >= 0 && k < K) table[k] = (uint16_t)i;
  }
  if (idx >= (size_t)npanels * nb * 64) return;
  const int l = (int)(idx % 64);
  const size_t pb = idx / 64;
  const int b = (int)(pb % nb), panel = (int)(pb / nb);
  const int n = panel * kQ4Panel + l % 16;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t word = 0;  // padding rows and columns: u = 0, met by x = 0 or dropped
    if (n < N) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = BR * b + 64 * j + 32 * h + 8 * (l / 16) + e;
          if (i >= K) continue;
          const int src = perm ? perm[i] : i;
          if (src < 0 || src >= K) continue;
          const uint32_t sw = qw[(size_t)(src >> 4) * N + n];
          word |= ((sw >> (2 * (src & 15))) & 3u) << (2 * q2_pos(h, e));
        }
    }
    out[idx * 4 + j] = word;
  }
}

// ---------------------------------------------------------------------------
// The fused product.
//
// A workgroup walks a contiguous run of panels; its 8 waves split every
// panel's blocks into contiguous, group-aligned ranges and keep kQ4Ring
// blocks in flight.  Each wave leaves its partial tile per panel in LDS; one
// barrier at the end, then the workgroup sums the waves and writes Y.
// NSC: groups that close in each block (BR / G: 1 .. 8), or 0 when a group
// spans several blocks (G > BR); one scale (and zero) load per group closed,
// one per block when NSC = 0.
// ---------------------------------------------------------------------------
// ZP: asymmetric form, w = (u - zero) * scale with an fp16 zero per (group,
// column) ("Quantization CUDA", tom-jerr.github.io, sections "量化粒度" and
// "Marlin 格式"); without it the offset is the fixed 8 of the symmetric codes.
template <int MT, int NSC, bool ZP, int BITS>
__global__ __launch_bounds__(kQ4Threads) void q4_mfma_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ Y, int M, int K, int N, int lg, int nb, int npanels, int pq, int pe,
    int packed_bytes) {
  // G = 2^lg (the entry points take powers of two only): group arithmetic by
  // shifts, with no integer divide ahead of the first load.
  const int G = 1 << lg;
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int BR = block_rows<BITS>();  // rows per block
  constexpr int SPB = BR / 32;            // MFMA steps per block
  static_assert(BITS == 4 || ZP, "2-bit codes come with zero points");
  const int rs = nb * BR + kQ4RowPad;                                  // halves per LDS row of X
  const int xhalves = rs * MT;                                          // halves of X in LDS
  _Float16* xa = reinterpret_cast<_Float16*>(smem);                     // [MT][octet][8], padded rows
  float* red = reinterpret_cast<float*>(smem + (size_t)xhalves * 2);  // [run][wave][MT][16]
  float* sg = red + kQ4MaxRun * kQ4Waves * MT * 16;  // [groups of nb * BR rows][8] group sums

  const int t = threadIdx.x, lane = t & 63;
  // Uniform across the wave: keeps the block range and cursors in scalar
  // registers and their branches scalar.
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Workgroups b and b + 8 run on the same XCD (dispatch is round-robin over
  // the 8 XCDs).  Each XCD takes a contiguous range of panel runs, so a
  // 128-byte line of a scale or zero row (64 columns: four panels) is
  // fetched into one XCD's L2, not into up to four.
  const int G8 = gridDim.x % 8 == 0 ? gridDim.x / 8 : 0;
  const int run = G8 ? (int)(blockIdx.x % 8) * G8 + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const SplitPart part = split_part(run, pq, pe);
  const int p_begin = part.begin, npr = part.count;

  // Blocks of this wave: a group-aligned contiguous range.
  constexpr int lBR = __builtin_ctz(BR);
  const int lbpg = lg > lBR ? lg - lBR : 0;  // log2(bpg)
  const int bpg = 1 << lbpg;
  const int nsplit = nb >> lbpg;
  const int blo = (wave * nsplit / kQ4Waves) * bpg, bhi = ((wave + 1) * nsplit / kQ4Waves) * bpg;
  const int nbw = bhi - blo;
  const int nitems = npr * nbw;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, packed_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (K >> lg) * N * 2);
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(ZP ? zeros : scales, (K >> lg) * N * 2);
  const int col = lane & 15;

  // Ring buffers: one 16-byte word quadruple, NL scale bits and (ZP) NL zero
  // bits per block.
  constexpr int NL = NSC == 0 ? 1 : NSC;  // scale loads per block
  constexpr int NZ = ZP ? NL : 1;
  u32x4 wb0, wb1, wb2, wb3;
  uint32_t sc0[NL], sc1[NL], sc2[NL], sc3[NL];
  uint32_t zp0[NZ], zp1[NZ], zp2[NZ], zp3[NZ];
  // Load cursor (panel of the run, block) walks the wave's blocks in order;
  // past the end it loads nothing (out-of-range offsets).
  int lp = nbw > 0 ? 0 : npr, lb = blo;
  int woff = ((p_begin * nb + blo) * 64 + lane) * 16;
  auto load_item = [&](u32x4& w, uint32_t (&sc)[NL], uint32_t (&zq)[NZ]) {
    const bool ok = lp < npr;
    const int n = (p_begin + lp) * kQ4Panel + col;
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int g = NSC == 0 ? (lb >> lbpg) : lb * NSC + k;  // the group closed k-th in the block
      const int off = (ok && n < N) ? (g * N + n) * 2 : kOutOfRange;
      sc[k] = __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0);
      if constexpr (ZP) zq[k] = __builtin_amdgcn_raw_buffer_load_b16(zr, off, 0, 0);
    }
    // The weights last: waiting for them covers the scales of the block.
    w = buffer_stream(wr, ok ? woff : kOutOfRange);
    woff += 1024;
    if (++lb == bhi) {
      lb = blo;
      ++lp;
      woff = (((p_begin + lp) * nb + blo) * 64 + lane) * 16;
    }
  };
  // Stage X through the row table of the packed weight: row k of X goes to
  // group-order row i = table[k], octet i / 8, position q4_pos(i % 8).  Rows
  // past K (block padding) and rows m >= M stay zero.  The loads of the first
  // round of chunks go out first, then the first kQ4Ring blocks of the weight
  // stream, so the scatter waits only for its own data.
  const int nchunk = K / 8;
  constexpr int CR = 2;  // chunks per thread per round
  // Buffer loads: chunks past K and rows past M read zero without a branch.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t tr = make_rsrc(Wp + (size_t)npanels * nb * 1024, K * 2);
  auto stage_load = [&](int c0, u32x4 (&pv)[CR], u32x4 (&xq)[CR][MT]) {
#pragma unroll
    for (int r = 0; r < CR; ++r) {
      const int ch = c0 + r * kQ4Threads;
      const bool ok = ch < nchunk;
      pv[r] = __builtin_amdgcn_raw_buffer_load_b128(tr, ok ? 16 * ch : kOutOfRange, 0, 0);
#pragma unroll
      for (int m = 0; m < MT; ++m)
        xq[r][m] = __builtin_amdgcn_raw_buffer_load_b128(
            xr, (ok && m < M) ? (m * K + 8 * ch) * 2 : kOutOfRange, 0, 0);
    }
  };
  auto stage_write = [&](int c0, const u32x4 (&pv)[CR], const u32x4 (&xq)[CR][MT]) {
#pragma unroll
    for (int r = 0; r < CR; ++r) {
      const int ch = c0 + r * kQ4Threads;
      if (ch >= nchunk) break;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = (int)((pv[r][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
        const int base = (i >> 3) * 8 + q4_pos(i & 7);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint32_t word = xq[r][m][j >> 1];
          const uint16_t bits = (j & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
          reinterpret_cast<uint16_t*>(xa)[m * rs + base] = bits;
        }
      }
    }
  };
  {
    u32x4 pv[CR], xq[CR][MT];
    stage_load(t, pv, xq);
    load_item(wb0, sc0, zp0);
    load_item(wb1, sc1, zp1);
    load_item(wb2, sc2, zp2);
    load_item(wb3, sc3, zp3);
    // Rows m < MT beyond K (block padding): zero.  The reduction tiles: zero.
    uint32_t* xz = reinterpret_cast<uint32_t*>(xa);
    const int padw = (rs - K) / 2;  // words per row past K
    for (int h = t; h < padw * MT; h += kQ4Threads) xz[(h / padw) * (rs / 2) + K / 2 + h % padw] = 0u;
    for (int r = t; r < kQ4MaxRun * kQ4Waves * MT * 16; r += kQ4Threads) red[r] = 0.0f;
    stage_write(t, pv, xq);
  }
  for (int c0 = t + CR * kQ4Threads; c0 < nchunk; c0 += CR * kQ4Threads) {
    u32x4 pv[CR], xq[CR][MT];
    stage_load(c0, pv, xq);
    stage_write(c0, pv, xq);
  }
  __syncthreads();

  // Group sums of the wave's own groups: sg[g][m] = sum of the G halves of
  // group g (group order: octets g G / 8 .. (g + 1) G / 8 - 1) in row m < MT.
  // Eight lanes share one sum: part p adds octets p, p + 8, ... with v_dot2
  // against ones, then a 3-step butterfly over the eight lanes (a fixed
  // order, so the result is bitwise reproducible).  Only this wave reads
  // these entries, after its own writes: no workgroup barrier.  Entries of
  // rows m >= MT are never written; they only meet output rows that are
  // never stored.
  {
    const h2 one2 = {(_Float16)1.0f, (_Float16)1.0f};
    const int octs = G >> 3, part = lane & 7;
    const int g0 = (blo * BR) >> lg, ng = (nbw * BR) >> lg;
    for (int task = lane >> 3; task < ng * MT; task += 8) {
      const int g = g0 + task / MT, m = task % MT;
      const _Float16* row = xa + (size_t)m * rs + (size_t)g * G;
      float acc = 0.0f;
      for (int o = part; o < octs; o += 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(row + 8 * o);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = dot2(as_h2(v[e]), one2, acc);
      }
      float sv[1] = {acc};
      bfly<1, 2, 0>(sv, lane);
      if (part == 0) sg[g * 8 + m] = sv[0];
    }
  }

  const int am = (lane & 15) < MT ? (lane & 15) : MT - 1, aq = lane >> 4;
  const _Float16* xrow = xa + (size_t)am * rs + aq * 8;
  f4 C0 = {0.0f, 0.0f, 0.0f, 0.0f}, C1 = C0, tot = C0;

  // One block: SPB MFMA steps (two chains) and the groups they close; at the
  // wave's last block of a panel its partial tile goes to LDS.
  int cp = 0, cb = blo;  // compute cursor: panel of the run, block
  // Operands of X, read one block ahead into the other of two buffers (X is
  // the same for every panel, so after a wave's last block comes blo).  The
  // ring below alternates the buffers, so no operand is ever copied.
  h8 xa0[SPB], xa1[SPB];
  if (nbw > 0) {
#pragma unroll
    for (int j = 0; j < SPB; ++j) xa0[j] = *reinterpret_cast<const h8*>(xrow + ((BR / 8) * blo + 4 * j) * 8);
  }
  auto compute = [&](const u32x4& w, const uint32_t (&sc)[NL], const uint32_t (&zq)[NZ],
                     const h8 (&a)[SPB], h8 (&nxt)[SPB]) {
    const int pi = cp, b = cb;
    const int bn = b + 1 == bhi ? blo : b + 1;
#pragma unroll
    for (int j = 0; j < SPB; ++j) nxt[j] = *reinterpret_cast<const h8*>(xrow + ((BR / 8) * bn + 4 * j) * 8);
    // MFMA step st of the block; the group it completes, if any, closes.
    // With whole groups in a block (NSC >= 1) the first two steps of a group
    // start their chains from the constant 0 operand, so nothing is zeroed at
    // a close; groups spanning blocks (NSC = 0) zero both chains at a close.
    constexpr int SPG = NSC == 0 ? SPB : SPB / NSC;  // steps per group (in the block)
    const f4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    auto mstep = [&](int st, const u32x4 bw) {
      const h8 bv = __builtin_bit_cast(h8, bw);
      const int ts = st % SPG;  // step within its group
      if constexpr (NSC == 0) {
        if (st & 1)
          C1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st], bv, C1, 0, 0, 0);
        else
          C0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st], bv, C0, 0, 0, 0);
      } else {
        if (ts == 0)
          C0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st], bv, zero4, 0, 0, 0);
        else if (ts == 1)
          C1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st], bv, zero4, 0, 0, 0);
        else if (ts & 1)
          C1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st], bv, C1, 0, 0, 0);
        else
          C0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[st], bv, C0, 0, 0, 0);
      }
      bool close;
      int k = 0, g;
      if constexpr (NSC == 0) {
        close = st == SPB - 1 && ((b + 1) & (bpg - 1)) == 0;
        g = b >> lbpg;
      } else {
        close = ts == SPG - 1;
        k = st / SPG;
        g = b * NSC + k;
      }
      if (close) {
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)sc[k]);
        // -offset * 2^-24: the codes sit in the products as u * 2^-24.
        float zoff = -8.0f / kTwo24;
        if constexpr (ZP) zoff = (float)__builtin_bit_cast(_Float16, (uint16_t)zq[k]) * (-1.0f / kTwo24);
        // Group sums of this lane's rows 4 (lane / 16) + r.
        const f4 S = *reinterpret_cast<const f4*>(sg + g * 8 + 4 * aq);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float c = SPG == 1 ? C0[r] : C0[r] + C1[r];
          tot[r] = __builtin_fmaf(s, __builtin_fmaf(S[r], zoff, c), tot[r]);
          if constexpr (NSC == 0) C0[r] = C1[r] = 0.0f;
        }
      }
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (BITS == 4) {
        mstep(j, q4_mfma_operand(w[j]));
      } else {
        mstep(2 * j, q2_mfma_operand<0>(w[j]));
        mstep(2 * j + 1, q2_mfma_operand<1>(w[j]));
      }
    }
    if (++cb == bhi) {
      // The wave's share of panel pi: rows 4 (lane / 16) + r, column lane % 16.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * (lane >> 4) + r;
        if (m < MT) red[((pi * kQ4Waves + wave) * MT + m) * 16 + col] = tot[r];
        tot[r] = 0.0f;
      }
      cb = blo;
      ++cp;
    }
  };
  auto step = [&](int q, u32x4& w, uint32_t (&sc)[NL], uint32_t (&zq)[NZ], const h8 (&a)[SPB],
                  h8 (&nxt)[SPB]) {
    if (q < nitems) compute(w, sc, zq, a, nxt);
    // Unconditional (out-of-range past the end), so the loads of every ring
    // slot keep one issue order and each wait covers just its own block.
    load_item(w, sc, zq);
  };
  for (int q = 0; q < nitems; q += kQ4Ring) {
    step(q, wb0, sc0, zp0, xa0, xa1);
    step(q + 1, wb1, sc1, zp1, xa1, xa0);
    step(q + 2, wb2, sc2, zp2, xa0, xa1);
    step(q + 3, wb3, sc3, zp3, xa1, xa0);
  }
  __syncthreads();
  for (int r = t; r < npr * MT * 16; r += kQ4Threads) {
    const int pi = r / (MT * 16), m = (r / 16) % MT, c = r % 16;
    const int n = (p_begin + pi) * kQ4Panel + c;
    const float* v = red + (pi * kQ4Waves * MT + m) * 16 + c;
    float sum = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kQ4Waves; ++w2) sum += v[w2 * MT * 16];
    if (m < M && n < N) Y[(size_t)m * N + n] = (_Float16)(sum * kTwo24);
  }
}

// ---------------------------------------------------------------------------
// Bit-exact check: each packed piece through q4_mfma_pairs back to signed
// codes in the original row order (perm), one thread per piece.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q4_unpack_kernel(const uint8_t* __restrict__ Wp,
                                                             const int* __restrict__ perm,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N, int nb, int npanels) {
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)npanels * nb * 64) return;
  const int l = (int)(idx % 64);
  const size_t pb = idx / 64;
  const int b = (int)(pb % nb), panel = (int)(pb / nb);
  const int n = panel * kQ4Panel + l % 16;
  if (n >= N) return;
  const u32x4 w = *reinterpret_cast<const u32x4*>(Wp + idx * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h2 pr[4];
    q4_mfma_pairs(w[j], pr);
    const int i0 = kQ4Block * b + 32 * j + 8 * (l / 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t bits = as_u32(pr[e]);
      const int ia = i0 + e, ib = i0 + e + 4;
      const int ka = ia < K ? (perm ? perm[ia] : ia) : -1, kb = ib < K ? (perm ? perm[ib] : ib) : -1;
      if (ka >= 0 && ka < K) codes[(size_t)ka * N + n] = (int8_t)((int)(bits & 0xFFFFu) - 8);
      if (kb >= 0 && kb < K) codes[(size_t)kb * N + n] = (int8_t)((int)(bits >> 16) - 8);
    }
  }
}

// 2-bit: each piece through q2_mfma_pairs back to the values u (0..3) in the
// original row order.
__global__ __launch_bounds__(kThreads) void q2_unpack_kernel(const uint8_t* __restrict__ Wp,
                                                             const int* __restrict__ perm,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N, int nb, int npanels) {
  constexpr int BR = block_rows<2>();
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (size_t)npanels * nb * 64) return;
  const int l = (int)(idx % 64);
  const size_t pb = idx / 64;
  const int b = (int)(pb % nb), panel = (int)(pb / nb);
  const int n = panel * kQ4Panel + l % 16;
  if (n >= N) return;
  const u32x4 w = *reinterpret_cast<const u32x4*>(Wp + idx * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      h2 pr[4];
      if (h == 0)
        q2_mfma_pairs<0>(w[j], pr);
      else
        q2_mfma_pairs<1>(w[j], pr);
      const int i0 = BR * b + 64 * j + 32 * h + 8 * (l / 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t bits = as_u32(pr[e]);
        const int ia = i0 + e, ib = i0 + e + 4;
        const int ka = ia < K ? (perm ? perm[ia] : ia) : -1, kb = ib < K ? (perm ? perm[ib] : ib) : -1;
        if (ka >= 0 && ka < K) codes[(size_t)ka * N + n] = (int8_t)(bits & 0xFFFFu);
        if (kb >= 0 && kb < K) codes[(size_t)kb * N + n] = (int8_t)(bits >> 16);
      }
    }
  }
}

hipError_t launch_q4_prepack(const int32_t* qw, const int32_t* perm, void* out, int K, int N, int G,
                             hipStream_t s) {
  const PanelPlan p = plan_q4(K, N, G);
  const size_t total = (size_t)p.npanels * p.u * 64;
  hipLaunchKernelGGL(q4_prepack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(qw), perm,
                     reinterpret_cast<uint32_t*>(out),
                     reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(out) + q4_block_bytes(p)),
                     reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(out) +
                                                 q4_fwd_table_offset(K, N)),
                     K, N, p.u, p.npanels);
  return hipGetLastError();
}

hipError_t launch_q4_unpack(const void* packed, const int32_t* perm, int8_t* codes, int K, int N,
                            int G, hipStream_t s) {
  const PanelPlan p = plan_q4(K, N, G);
  const size_t total = (size_t)p.npanels * p.u * 64;
  hipLaunchKernelGGL(q4_unpack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint8_t*>(packed), perm, codes, K,
                     N, p.u, p.npanels);
  return hipGetLastError();
}

hipError_t launch_q2_prepack(const int32_t* qw, const int32_t* perm, void* out, int K, int N, int G,
                             hipStream_t s) {
  const PanelPlan p = plan_q2(K, N, G);
  const size_t total = (size_t)p.npanels * p.u * 64;
  hipLaunchKernelGGL(q2_prepack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(qw), perm,
                     reinterpret_cast<uint32_t*>(out),
                     reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(out) + q4_block_bytes(p)), K,
                     N, p.u, p.npanels);
  return hipGetLastError();
}

hipError_t launch_q2_unpack(const void* packed, const int32_t* perm, int8_t* codes, int K, int N,
                            int G, hipStream_t s) {
  const PanelPlan p = plan_q2(K, N, G);
  const size_t total = (size_t)p.npanels * p.u * 64;
  hipLaunchKernelGGL(q2_unpack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint8_t*>(packed), perm, codes, K,
                     N, p.u, p.npanels);
  return hipGetLastError();
}

template <int MT, int NSC, bool ZP, int BITS>
static hipError_t launch_q4_t(const void* X, const void* packed, const void* scales,
                              const void* zeros, void* Y, int M, int K, int N, int G,
                              const PanelPlan& p, hipStream_t s) {
  constexpr int BR = block_rows<BITS>();
  const int cus = device_cus();
  int grid = p.npanels < cus ? p.npanels : cus;
  if ((p.npanels + grid - 1) / grid > kQ4MaxRun) grid = (p.npanels + kQ4MaxRun - 1) / kQ4MaxRun;
  // Group sums: one entry per group of the padded rows p.u * BR (a ragged
  // last block closes groups past K / G, whose rows are all padding).
  const size_t ngroups = ((size_t)p.u * BR + G - 1) / G;
  const size_t lds = ((size_t)p.u * BR + kQ4RowPad) * MT * 2 +
                     (size_t)kQ4MaxRun * kQ4Waves * MT * 16 * 4 + ngroups * 8 * 4;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&q4_mfma_kernel<MT, NSC, ZP, BITS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((q4_mfma_kernel<MT, NSC, ZP, BITS>), dim3(grid), dim3(kQ4Threads), lds, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                     reinterpret_cast<const _Float16*>(scales),
                     reinterpret_cast<const _Float16*>(zeros), reinterpret_cast<_Float16*>(Y), M,
                     K, N, __builtin_ctz((unsigned)G), p.u, p.npanels, p.npanels / grid, p.npanels % grid,
                     (int)q4_block_bytes(p));
  return hipGetLastError();
}

// Groups closed per block (NSC): BR / G for G <= BR, 0 for groups spanning
// several blocks.
template <int MT, bool ZP, int BITS>
static hipError_t launch_q4_zp(const void* X, const void* packed, const void* scales,
                               const void* zeros, void* Y, int M, int K, int N, int G,
                               const PanelPlan& p, hipStream_t s) {
  constexpr int BR = block_rows<BITS>();
  const int nsc = G > BR ? 0 : BR / G;
  if constexpr (BITS == 2) {
    if (nsc == 8) return launch_q4_t<MT, 8, ZP, BITS>(X, packed, scales, zeros, Y, M, K, N, G, p, s);
  }
  if (nsc == 4) return launch_q4_t<MT, 4, ZP, BITS>(X, packed, scales, zeros, Y, M, K, N, G, p, s);
  if (nsc == 2) return launch_q4_t<MT, 2, ZP, BITS>(X, packed, scales, zeros, Y, M, K, N, G, p, s);
  if (nsc == 1) return launch_q4_t<MT, 1, ZP, BITS>(X, packed, scales, zeros, Y, M, K, N, G, p, s);
  return launch_q4_t<MT, 0, ZP, BITS>(X, packed, scales, zeros, Y, M, K, N, G, p, s);
}

template <int MT, int BITS>
static hipError_t launch_q4_mt(const void* X, const void* packed, const void* scales,
                               const void* zeros, void* Y, int M, int K, int N, int G,
                               const PanelPlan& p, hipStream_t s) {
  if constexpr (BITS == 2)
    return launch_q4_zp<MT, true, 2>(X, packed, scales, zeros, Y, M, K, N, G, p, s);
  else
    return zeros ? launch_q4_zp<MT, true, 4>(X, packed, scales, zeros, Y, M, K, N, G, p, s)
                 : launch_q4_zp<MT, false, 4>(X, packed, scales, zeros, Y, M, K, N, G, p, s);
}

template <int BITS>
static hipError_t launch_blocks(const void* X, const void* packed, const void* scales,
                                const void* zeros, void* Y, int M, int K, int N, int G,
                                hipStream_t s) {
  constexpr int BR = block_rows<BITS>();
  const PanelPlan p = plan_blocks(K, N, BR, BITS == 4);
  const int mtmax = max_mt(K, BR);
  for (int m0 = 0; m0 < M; m0 += mtmax) {
    const int mc = (M - m0) < mtmax ? (M - m0) : mtmax;
    const int mt = mc == 1 ? 1 : (mc == 2 ? 2 : (mc <= 4 ? 4 : 8));
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)m0 * K * 2;
    void* Yc = reinterpret_cast<char*>(Y) + (size_t)m0 * N * 2;
    hipError_t e;
    switch (mt) {
      case 1: e = launch_q4_mt<1, BITS>(Xc, packed, scales, zeros, Yc, mc, K, N, G, p, s); break;
      case 2: e = launch_q4_mt<2, BITS>(Xc, packed, scales, zeros, Yc, mc, K, N, G, p, s); break;
      case 4: e = launch_q4_mt<4, BITS>(Xc, packed, scales, zeros, Yc, mc, K, N, G, p, s); break;
      default: e = launch_q4_mt<8, BITS>(Xc, packed, scales, zeros, Yc, mc, K, N, G, p, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_q4_group(const void* X, const void* packed, const void* scales,
                           const void* zeros, void* Y, void* ws, int M, int K, int N, int G,
                           hipStream_t s) {
  if (M > kQ4TiledMinRows) return launch_q4_tiled(X, packed, scales, zeros, Y, ws, M, K, N, G, s);
  return launch_blocks<4>(X, packed, scales, zeros, Y, M, K, N, G, s);
}

hipError_t launch_q2_group(const void* X, const void* packed, const void* scales,
                           const void* zeros, void* Y, int M, int K, int N, int G, hipStream_t s) {
  return launch_blocks<2>(X, packed, scales, zeros, Y, M, K, N, G, s);
}

}  // namespace wq
