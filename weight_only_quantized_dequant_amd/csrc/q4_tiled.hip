// 4-bit group-wise GEMM for more rows of X (5 .. 64 per launch), reading the
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
//     codes in a packed word).  A wave stages one row of X in LDS with
//     coalesced loads, reads 64 octets of original row numbers from the
//     forward row table, and gathers from LDS.  Padding rows past K are
//     zero; rows of the last tile past M are not written, and the GEMM's
//     loads of them fall out of range.
// (2) The GEMM.  A workgroup takes a run of at most 3 panels and every row
//     of the launch (one to four 16-row tiles); each of its 8 waves walks a
//     contiguous share of the 128-row blocks with a ring of blocks in
//     flight.  Per block a wave issues few, wide loads (the vector memory
//     path's per-instruction cost bounds this kernel): its X operands (1 KB
//     per tile and step), one 16-byte piece of every panel's block, and one
//     8-byte piece of the block's scale (and zero) rows, whose values reach
//     the lanes that need them through cross-lane permutes.  Every operand
//     is read through a buffer range that ends where the wave's share ends.
//     Per run of rows that shares a group (a block, or 64 / 32 rows):
//       C1 = 2^-24 * c * sum_i x_i   (matrix cores, a constant operand c:
//                                     -8 for the symmetric codes, 1 with zeros)
//       C  = D + 2^-24 * sum_i x_i u_i,  D = C1, or -z * C1 with zeros
//       tot += scale * C
//     so C = 2^-24 * sum_i x_i (u_i - z), the codes entering as exact fp16
//     subnormals.  At the end the 8 waves' tiles are added in LDS in a fixed
//     order and Y = 2^24 * tot.
#include "q4_layout.hpp"
#include "wq_internal.h"

namespace wq {

constexpr int kQTThreads = 512;
constexpr int kQTWaves = kQTThreads / 64;
constexpr int kQTMaxRun = 3;    // panels per workgroup at most, one row group
constexpr int kQTWideRun = 6;   // the same with two row groups of two tiles

int q4_tiled_kp(int K) { return (K + kQ4Block - 1) / kQ4Block * kQ4Block; }

// Workspace: the operand-order copy of X, mbt 16-row tiles of Kp halves.
static size_t q4_xo_bytes(int mbt, int Kp) { return (size_t)mbt * 16 * Kp * 2; }
size_t q4_tiled_workspace_bytes(int M, int K) {
  if (M <= kQ4TiledMinRows) return 0;
  return q4_xo_bytes((M + 15) / 16, q4_tiled_kp(K));
}

// (1) One wave per (row m < M, range r of 64 octets of
// group-order rows).  The wave copies row m of X into LDS (coalesced), then
// lane l takes octet o = 64 r + l (group-order rows 8 o .. 8 o + 7): their
// original rows from the forward table (one 16-byte load, issued first),
// the 8 values read from LDS, and one 16-byte store of the operand piece
// (step o / 4, lane m % 16 + 16 (o % 4) of tile m / 16).  Padding rows give
// zeros.
constexpr int kQXThreads = 64;
constexpr int kQXBatch = 8 * 64 * 8;  // halves of X per batch: 8 pieces of 16 bytes per lane
__global__ __launch_bounds__(kQXThreads) void q4_xgather_kernel(const _Float16* __restrict__ X,
                                                                const uint16_t* __restrict__ fwd,
                                                                _Float16* __restrict__ Xo, int M,
                                                                int K, int Kp, int mbt) {
  extern __shared__ uint16_t xrow[];  // K rounded up to kQXBatch halves
  const int lane = threadIdx.x;
  const int m = blockIdx.y;
  const int o = blockIdx.x * 64 + lane;
  // Loads past the ranges return zeros: the table past Kp rows, and the
  // whole row when m >= M.
  const __amdgpu_buffer_rsrc_t tr = make_rsrc(fwd, Kp * 2);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + (size_t)(m < M ? m : 0) * K, m < M ? K * 2 : 0);
  const u32x4 tv = __builtin_amdgcn_raw_buffer_load_b128(tr, o * 16, 0, 0);
  // Every load of a batch is issued before its LDS writes.
  for (int i0 = 0; i0 < K; i0 += kQXBatch) {
    u32x4 t[8];
#pragma unroll
    for (int b = 0; b < 8; ++b)
      t[b] = __builtin_amdgcn_raw_buffer_load_b128(xr, (i0 + (b * 64 + lane) * 8) * 2, 0, 0);
#pragma unroll
    for (int b = 0; b < 8; ++b)
      *reinterpret_cast<u32x4*>(xrow + i0 + (b * 64 + lane) * 8) = t[b];
  }
  __syncthreads();
  uint32_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = (int)((tv[e >> 1] >> (16 * (e & 1))) & 0xFFFFu);
    const uint32_t x = xrow[k < K ? k : K - 1];
    v[e] = k < K ? x : 0u;  // 0xFFFF: a padding row
  }
  // Operand order 0 4 1 5 2 6 3 7: half 2 j holds row j, half 2 j + 1 row j + 4.
  const u32x4 op = {v[0] | (v[4] << 16), v[1] | (v[5] << 16), v[2] | (v[6] << 16),
                    v[3] | (v[7] << 16)};
  if (o < Kp / 8) {
    const int step = o >> 2, mb = m >> 4;
    *reinterpret_cast<u32x4*>(Xo + (((size_t)step * mbt + mb) * 64 + (m & 15) + 16 * (o & 3)) * 8) =
        op;
  }
}

// (2) MB: 16-row tiles per workgroup; CPB: groups per block (1 for groups of
// 128 rows or more, else 128 / G); BD: blocks in flight per wave; RUN:
// panels per workgroup at most.  blockIdx.y picks the row group: tiles
// MB y .. MB y + MB - 1 of the launch's M rows.
template <int MB, int CPB, bool ZP, int BD, int RUN>
__global__ __launch_bounds__(kQTThreads) void q4_tiled_kernel(
    const _Float16* __restrict__ Xo, const uint8_t* __restrict__ Wp,
    const _Float16* __restrict__ scales, const _Float16* __restrict__ zeros,
    _Float16* __restrict__ Y, int M, int mb0, int mbt, int N, int ngroups, int lg, int nb, int pq,
    int pe) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
  constexpr int MT = 16 * MB;
  constexpr int SPC = 4 / CPB;  // MFMA steps per group run
  static_assert(4 * RUN * CPB <= 64, "a block's scale table is one 8-byte piece per lane");
  __shared__ float red[RUN * kQTWaves * MT * 16];  // [run][wave][MT][16]
  // This workgroup's row group.
  M -= MT * (int)blockIdx.y;
  mb0 += MB * (int)blockIdx.y;
  Y += (size_t)MT * blockIdx.y * N;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  // Each XCD (workgroups b = x mod 8) takes a contiguous range of panel runs,
  // so a 128-byte line of a scale or zero row (four panels) is fetched into
  // one XCD's L2.  With gridDim.x a multiple of 8 the row groups of a run
  // share the XCD too, and so the run's weight in that L2.
  const int G8 = gridDim.x % 8 == 0 ? gridDim.x / 8 : 0;
  const int run = G8 ? (int)(blockIdx.x % 8) * G8 + (int)(blockIdx.x / 8) : (int)blockIdx.x;
  const SplitPart part = split_part(run, pq, pe);
  const int p_begin = part.begin, npr = part.count;
  // This wave's blocks [bw0, bw0 + nbw).  The share a wave takes rotates
  // with the workgroup, so the workgroups of an XCD do not all read the same
  // rows of X at the same moment.
  const int share = (wave + run) % kQTWaves;
  const int bw0 = share * nb / kQTWaves, nbw = (share + 1) * nb / kQTWaves - bw0;
  const int col = lane & 15;

  // Buffer ranges that end with this wave's share.
  const int xblock = 4 * mbt * 1024;  // X operand bytes of one block, all tiles
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(reinterpret_cast<const char*>(Xo) + (size_t)bw0 * xblock, nbw * xblock);
  __amdgpu_buffer_rsrc_t wr[RUN];
#pragma unroll
  for (int p = 0; p < RUN; ++p) {
    const int panel = p < npr ? p_begin + p : 0;
    wr[p] = make_rsrc(Wp + ((size_t)panel * nb + bw0) * 1024, p < npr ? nbw * 1024 : 0);
  }
  // Scale (and zero) rows of a block: CPB groups x 16 RUN columns (the run's
  // panels) as one table, lane l holding halves 4 l .. 4 l + 3: group
  // l / (4 RUN), columns 4 (l % (4 RUN)) .. +3 of the run.  Lanes past the
  // table, and columns past N (N % 4 == 0: a piece never straddles it), read
  // zeros.
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, ngroups * N * 2);
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(ZP ? zeros : scales, ngroups * N * 2);
  const int tcol = p_begin * kQ4Panel + 4 * (lane % (4 * RUN));
  const bool tlive = lane < 4 * RUN * CPB && tcol < N;
  const int tlane = (lane / (4 * RUN)) * N * 2 + tcol * 2;
  // Where this lane finds its column's value for panel p, group c of a
  // block: lane (16 RUN c + 16 p + col) / 4, dword (col / 2) % 2, half
  // col % 2.
  const int hshift = 16 * (col & 1);
  const bool hi = (col & 2) != 0;
  const int xlane = lane * 16, wlane = lane * 16;

  struct Block {
    u32x4 a[4][MB];        // X operands: step, tile
    u32x4 w[RUN];          // weight words of the 4 steps, per panel
    u32x2v sc;             // this lane's piece of the scale table
    u32x2v zq;             // and of the zero table (ZP)
  };
  // Loads of this wave's block j.  The ring asks for blocks past the share;
  // those loads take the share's last block again (their values are never
  // used), so every address stays inside the wave's ranges.  A wave with no
  // share has empty ranges: its loads all return zeros.
  auto clampj = [&](int jr) { return jr < nbw ? jr : (nbw > 0 ? nbw - 1 : 0); };
  // Lanes whose row of the tile is past M read out of range (zeros, and no
  // memory request): a partial tile moves only its live rows.
  auto load_x = [&](int jr, Block& q, int mb) {
    const int j = clampj(jr);
    const int xo = 16 * mb + col < M ? xlane + mb * 1024 : kOutOfRange;
#pragma unroll
    for (int st = 0; st < 4; ++st)
      q.a[st][mb] = __builtin_amdgcn_raw_buffer_load_b128(
          xr, xo, (4 * j + st) * mbt * 1024 + mb0 * 1024, 0);
  };
  auto load_wt = [&](int jr, Block& q) {
    const int j = clampj(jr);
#pragma unroll
    for (int p = 0; p < RUN; ++p)
      q.w[p] = __builtin_amdgcn_raw_buffer_load_b128(wr[p], wlane, j * 1024, 2);
    // First group of the block; the whole offset is in the lane's offset,
    // so groups past the last one (padding rows) fall out of range.
    const int g0 = ((bw0 + j) * kQ4Block) >> lg;  // G = 2^lg
    const int so = tlive ? tlane + g0 * N * 2 : kOutOfRange;
    q.sc = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(sr, so, 0, 0));
    if constexpr (ZP)
      q.zq = __builtin_bit_cast(u32x2v, __builtin_amdgcn_raw_buffer_load_b64(zr, so, 0, 0));
  };
  auto load = [&](int jr, Block& q) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) load_x(jr, q, mb);
    load_wt(jr, q);
  };
  // This lane's column value of panel p, group c from a block's table.
  auto table_value = [&](const u32x2v& tbl, int p, int c) {
    const int src = ((16 * RUN * c + 16 * p + col) >> 2) * 4;
    const uint32_t d0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)tbl[0]);
    const uint32_t d1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)tbl[1]);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((hi ? d1 : d0) >> hshift));
  };

  f4 tot[RUN][MB];
#pragma unroll
  for (int p = 0; p < RUN; ++p)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) tot[p][mb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
  // The constant operand of the row sums: -8 * 2^-24 (fp16 subnormal bits
  // 0x8008) for the symmetric codes, 2^-24 (0x0001) with zeros.
  const uint32_t cbits = ZP ? 0x00010001u : 0x80088008u;
  const h8 cop = __builtin_bit_cast(h8, u32x4{cbits, cbits, cbits, cbits});
  const f4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  // One block.  Every panel slot runs, also past the run (its weights and
  // scales read as zero, its tile is never stored): no branch between an
  // MFMA and the first read of its result.
  auto compute = [&](const Block& q) {
#pragma unroll
    for (int c = 0; c < CPB; ++c) {
      f4 c1[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        f4 r = zero4;
#pragma unroll
        for (int st = c * SPC; st < (c + 1) * SPC; ++st)
          r = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, q.a[st][mb]), cop, r,
                                                     0, 0, 0);
        c1[mb] = r;
      }
#pragma unroll
      for (int p = 0; p < RUN; ++p) {
        h8 b[SPC];
#pragma unroll
        for (int i = 0; i < SPC; ++i)
          b[i] = __builtin_bit_cast(h8, q4_mfma_operand(q.w[p][c * SPC + i]));
        const float sv = table_value(q.sc, p, c);
        float nz = 1.0f;
        if constexpr (ZP) nz = -table_value(q.zq, p, c);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          f4 r = c1[mb];
          if constexpr (ZP) r *= nz;
#pragma unroll
          for (int i = 0; i < SPC; ++i)
            r = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, q.a[c * SPC + i][mb]),
                                                       b[i], r, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) tot[p][mb][e] = __builtin_fmaf(sv, r[e], tot[p][mb][e]);
        }
      }
    }
  };

  if constexpr (BD > 0) {
    // The ring: slot i holds block j + i.  Loads are issued in block order
    // and scheduling barriers keep them so, so the oldest slot's loads are
    // always the first outstanding ones and each wait before a compute
    // covers only its own block.
    Block q[BD];
#pragma unroll
    for (int i = 0; i < BD; ++i) {
      load(i, q[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    int j = 0;
    for (; j + BD < nbw; j += BD) {
#pragma unroll
      for (int i = 0; i < BD; ++i) {
        compute(q[i]);
        load(j + BD + i, q[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int i = 0; i < BD; ++i)
      if (j + i < nbw) compute(q[i]);
  } else {
    // Three or four tiles: one block's X fills the registers, so the next
    // block streams in tile by tile.  The weights and tables of block j + 1
    // are requested as soon as block j's are unpacked, and the X of tile mb
    // of block j + 1 right after tile mb of block j is done.
    // The prologue issues block 0 in the loop's order (weights and tables,
    // then X tile by tile), so every wait in the loop counts the same loads.
    Block q;
    load_wt(0, q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      load_x(0, q, mb);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int j = 0; j < nbw; ++j) {
      h8 b[RUN][4];
      float sv[RUN][CPB], nz[RUN][CPB];
#pragma unroll
      for (int p = 0; p < RUN; ++p) {
#pragma unroll
        for (int st = 0; st < 4; ++st) b[p][st] = __builtin_bit_cast(h8, q4_mfma_operand(q.w[p][st]));
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
          sv[p][c] = table_value(q.sc, p, c);
          nz[p][c] = ZP ? -table_value(q.zq, p, c) : 1.0f;
        }
      }
      load_wt(j + 1, q);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
          f4 c1 = zero4;
#pragma unroll
          for (int st = c * SPC; st < (c + 1) * SPC; ++st)
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, q.a[st][mb]), cop,
                                                        c1, 0, 0, 0);
#pragma unroll
          for (int p = 0; p < RUN; ++p) {
            f4 r = c1;
            if constexpr (ZP) r *= nz[p][c];
#pragma unroll
            for (int st = c * SPC; st < (c + 1) * SPC; ++st)
              r = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, q.a[st][mb]),
                                                         b[p][st], r, 0, 0, 0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              tot[p][mb][e] = __builtin_fmaf(sv[p][c], r[e], tot[p][mb][e]);
          }
        }
        load_x(j + 1, q, mb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

#pragma unroll
  for (int p = 0; p < RUN; ++p)
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

// Blocks in flight per wave: what fits the registers without spilling.
// 0: the tile-by-tile stream of one block (three or four tiles).  One block
// of a wide run is 14 KB per wave, so one in flight per wave already fills
// the CU's request window.
constexpr int q4_tiled_depth(int MB, int CPB, bool ZP, int RUN) {
  return (void)ZP, MB >= 3 ? 0 : RUN > kQTMaxRun ? 1 : (MB == 1 || CPB == 1) ? 2 : 1;
}
// Tiles per launch at most: groups of 64 and 32 close 2 and 4 times per
// block, and their extra row sums and scale values no longer fit the
// registers with four (three) tiles.
constexpr int q4_tiled_max_tiles(int G) { return G == 32 ? 2 : G == 64 ? 3 : 4; }

// RG row groups of MB tiles, runs of at most RUN panels: as many runs as
// fill the CUs with RG workgroups each, fewer if a run would pass RUN.
template <int MB, int CPB, bool ZP, int RUN, int RG>
static hipError_t launch_q4_tiled_t(const _Float16* Xo, const uint8_t* Wp, const _Float16* scales,
                                    const _Float16* zeros, _Float16* Y, int M, int mb0, int mbt,
                                    int K, int N, int G, hipStream_t s) {
  constexpr int BD = q4_tiled_depth(MB, CPB, ZP, RUN);
  const int nb = q4_tiled_kp(K) / kQ4Block, npanels = (N + kQ4Panel - 1) / kQ4Panel;
  const int cus = device_cus() / RG;
  int grid = npanels < cus ? npanels : cus;
  if ((npanels + grid - 1) / grid > RUN) grid = (npanels + RUN - 1) / RUN;
  hipLaunchKernelGGL((q4_tiled_kernel<MB, CPB, ZP, BD, RUN>), dim3(grid, RG), dim3(kQTThreads), 0, s,
                     Xo, Wp, scales, zeros, Y, M, mb0, mbt, N, K / G, __builtin_ctz((unsigned)G), nb, npanels / grid,
                     npanels % grid);
  return hipGetLastError();
}

template <int MB, int CPB, int RUN, int RG>
static hipError_t launch_q4_tiled_z(const _Float16* Xo, const uint8_t* Wp, const _Float16* scales,
                                    const _Float16* zeros, _Float16* Y, int M, int mb0, int mbt,
                                    int K, int N, int G, hipStream_t s) {
  return zeros ? launch_q4_tiled_t<MB, CPB, true, RUN, RG>(Xo, Wp, scales, zeros, Y, M, mb0, mbt, K,
                                                          N, G, s)
               : launch_q4_tiled_t<MB, CPB, false, RUN, RG>(Xo, Wp, scales, zeros, Y, M, mb0, mbt, K,
                                                           N, G, s);
}

// One to two tiles: one row group, runs of up to 3 panels.  Three or four
// tiles with groups of 128 rows or more: two row groups of two tiles and
// runs of up to 6 panels, so a workgroup reads half of X (X, read by every
// workgroup, is most of what a workgroup loads at 64 rows); the two row
// groups of a run take its weight from one L2.  (With groups of 64 the
// second group per block does not fit the registers of a wide run.)
template <int NT>
static hipError_t launch_q4_tiled_mb(const _Float16* Xo, const uint8_t* Wp, const _Float16* scales,
                                     const _Float16* zeros, _Float16* Y, int M, int mb0, int mbt,
                                     int K, int N, int G, hipStream_t s) {
  if (G == 32) {
    if constexpr (NT > q4_tiled_max_tiles(32)) return hipErrorInvalidValue;
    else return launch_q4_tiled_z<NT, 4, kQTMaxRun, 1>(Xo, Wp, scales, zeros, Y, M, mb0, mbt, K, N, G, s);
  }
  if (G == 64) {
    if constexpr (NT > q4_tiled_max_tiles(64)) return hipErrorInvalidValue;
    else return launch_q4_tiled_z<NT, 2, kQTMaxRun, 1>(Xo, Wp, scales, zeros, Y, M, mb0, mbt, K, N, G, s);
  }
  if constexpr (NT <= 2)
    return launch_q4_tiled_z<NT, 1, kQTMaxRun, 1>(Xo, Wp, scales, zeros, Y, M, mb0, mbt, K, N, G, s);
  else
    return launch_q4_tiled_z<2, 1, kQTWideRun, 2>(Xo, Wp, scales, zeros, Y, M, mb0, mbt, K, N, G, s);
}

hipError_t launch_q4_tiled(const void* X, const void* packed, const void* scales,
                           const void* zeros, void* Y, void* ws, int M, int K, int N, int G,
                           hipStream_t s) {
  const int Kp = q4_tiled_kp(K);
  const int mbt = (M + 15) / 16;
  const uint8_t* Wp = reinterpret_cast<const uint8_t*>(packed);
  const uint16_t* fwd = reinterpret_cast<const uint16_t*>(Wp + q4_fwd_table_offset(K, N));
  _Float16* Xo = reinterpret_cast<_Float16*>(ws);
  // Rows past M are never read (the GEMM's loads of them fall out of range),
  // so only the M live rows are gathered.
  hipLaunchKernelGGL(q4_xgather_kernel, dim3((Kp / 8 + 63) / 64, M), dim3(kQXThreads),
                     (size_t)((K + kQXBatch - 1) / kQXBatch) * kQXBatch * 2, s,
                     reinterpret_cast<const _Float16*>(X), fwd, Xo, M, K, Kp, mbt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const _Float16* sc = reinterpret_cast<const _Float16*>(scales);
  const _Float16* zp = reinterpret_cast<const _Float16*>(zeros);
  const int rows = 16 * q4_tiled_max_tiles(G);
  for (int m0 = 0; m0 < M; m0 += rows) {
    const int mc = M - m0 < rows ? M - m0 : rows;
    _Float16* Yc = reinterpret_cast<_Float16*>(Y) + (size_t)m0 * N;
    const int mb0 = m0 / 16;
    switch ((mc + 15) / 16) {
      case 1: e = launch_q4_tiled_mb<1>(Xo, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
      case 2: e = launch_q4_tiled_mb<2>(Xo, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
      case 3: e = launch_q4_tiled_mb<3>(Xo, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
      default: e = launch_q4_tiled_mb<4>(Xo, Wp, sc, zp, Yc, mc, mb0, mbt, K, N, G, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
