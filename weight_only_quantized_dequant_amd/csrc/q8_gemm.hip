// Group-wise symmetric int8 weight-only GEMM for many rows of X, on the
// matrix cores.  Same product and same packed weight as q8_group.hip:
//
//   Y[m, n] = sum_g scale[g, n] * sum_{k in group g} X[m, k] * q[k, n]
//
// ("Quantization CUDA", tom-jerr.github.io, section "Int8 Weight Only
// Quantization": Y = X.(Wint*Sw) evaluated as (X.Wint)*Sw; the fused kernel of
// "融合反量化与GEMM：LLM推理的CUDA内核优化实践", zingnex.cn, sections "核心优化思路"
// and "技术实现细节": tiles of the int8 weight are dequantised on chip and never
// written back as floating point, one fp32 scale per 128 rows of K per column).
//
// Tiles.  A workgroup (4 waves) owns a 32 x 128 tile of Y and walks K in
// stages of 128 rows.  Per stage, direct-to-LDS buffer loads bring the X tile
// (fp16, 32 x 128), the int8 codes of the weight tile (128 rows x 128
// columns: 16 pieces of each of 64 column pairs of the packed layout, 8 rows
// x 2 columns per piece) and the scale rows of the stage's groups into a ring
// of kStages slots (75 KB: two workgroups fit on a CU).  Each wave builds its
// v_mfma_f32_16x16x32_f16 operands for a 16 x 64 sub-tile in registers,
// straight from the int8 stage: a piece is the 8 rows of one k32 octet for
// two columns, and one v_perm_b32 per word turns a column's two code bytes
// into two zero-exponent fp16s (the exact subnormals u 2^-24, u = q + 128),
// so one 16-byte LDS read gives the operands of two columns.  One more
// matrix-core product per k32 step against a constant operand of 128 2^-24
// gives the offset term.  Each wave keeps the current group's sums
// and a running total; at the end of a group the total takes
// (sums - offset term) * scale in fp32 and the next group starts from zero,
// so the products are exact and every rounding is an fp32 one, as in the
// small-batch kernel.  The result is scaled by 2^24 and rounded once to
// fp16.
//
// X rows of a stage are 256 bytes, 16 chunks of 16; chunk c of row r sits at
// position c ^ (r % 16), which keeps the 16 rows of one fragment read on
// distinct LDS banks.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kBM = 32, kBN = 128, kBK = 128, kStages = 3, kThreadsG = 256;
constexpr int kRowA = kBK * 2;                   // 256 bytes: one fp16 row of X per stage
constexpr int kStageA = kBM * kRowA;             // X tile, fp16 [m][k], 16 KB
constexpr int kStageB = kBK * kBN;               // codes: 128 rows x 8 chunks of 16 bytes
constexpr int kStageS = 1024;                    // two scale rows of 128 columns
constexpr int kStage = kStageA + kStageB + kStageS;
constexpr int kLoads = 6;                        // direct-to-LDS loads per stage per wave

// X rows of a stage are 16 chunks of 16 bytes; chunk c of row r sits at
// position c ^ (r % 16), so the 16 rows of one fragment read hit distinct
// LDS banks.
__device__ __forceinline__ int swz(int row, int c) { return c ^ (row & 15); }

}  // namespace

// Codes of a stage in LDS: piece b (rows 8 b .. 8 b + 7 of the stage,
// b = 0..15) of the tile's column pair p (0..63) sits at slot
// 16 p + (b ^ (p % 16)).  A direct-to-LDS load writes 64 consecutive slots:
// 4 pairs x 16 pieces, i.e. four 256-byte runs of the packed weight.  The
// swizzle keeps the 16 lanes of one fragment read (16 pairs, one piece
// each) on distinct banks.
//
// Fragments.  Lane l of a wave with columns w0 .. w0 + 63 (pairs w0 / 2 ..)
// takes, for the k32 step h and half H (0, 1), piece 4 h + l / 16 of pair
// w0 / 2 + 16 H + l % 16: the 8 rows 32 h + 8 (l / 16) + e of two columns.
// Column c of it goes to the matrix-core operand of block 2 H + c, so block
// 2 H + c, operand column t holds weight column w0 + 32 H + 2 t + c; the
// transposed result then gives lane l, per half, the 8 consecutive columns
// w0 + 32 H + 8 (l / 16) + 2 r + c (r = 0..3, c = 0, 1) of one row.
// Split K (S > 1): workgroup b takes K slice b % S (S divides 8, so with
// S = 8 every workgroup of an XCD reads the same slice of X) and writes its
// fp32 partial tile, still in units of 2^-24, to ws [S][M][N]; a second
// launch adds the slices in order and rounds once.  Slices are whole groups.
__global__ __launch_bounds__(kThreadsG, 2) void q8_gemm_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const float* __restrict__ scales, _Float16* __restrict__ Y, float* __restrict__ ws, int M,
    int K, int N, int G, int KB, int mtiles, int ntiles, int S) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStage];

  // Workgroups b and b + 8 run on the same XCD: the M tiles that share a
  // column tile of the weight are placed 8 apart.
  const int slice = (int)blockIdx.x % S;
  const int bid = (int)blockIdx.x / S;
  const int grp = bid / (8 * mtiles), rr = bid % (8 * mtiles);
  const int mt = rr / 8, nt = grp * 8 + (rr % 8);
  if (nt >= ntiles) return;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nkt = (K + kBK - 1) / kBK;   // stages of all of K
  const int kt0 = slice * nkt / S;       // this slice's stages [kt0, kt0 + nk)
  const int nk = (slice + 1) * nkt / S - kt0;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, K * N);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (K / G) * N * 4);

  // X: load t of wave w fills stage rows 4 (4 w + t) .. + 3; lane l brings
  // row 4 (4 w + t) + l / 16, chunk position l % 16.
  int a_off[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int row = 4 * (2 * wave + t) + (lane >> 4);
    a_off[t] = m0 + row < M ? (m0 + row) * K * 2 + 16 * swz(row, lane & 15) : -1;
  }
  // Codes: load t of wave w fills slots 64 (4 w + t) .. + 63, i.e. pair
  // p = 4 (4 w + t) + l / 16 of the tile, the piece that slot 16 p + l % 16
  // holds: b = (l % 16) ^ (p % 16), with p % 16 = 4 t + l / 16.
  int b_off[4], b_sw[4];
  bool b_live[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int pg = n0 / 2 + 4 * (4 * wave + t) + (lane >> 4);
    b_live[t] = pg < N / 2;
    b_off[t] = b_live[t] ? pg * KB * 16 : 0;
    b_sw[t] = (lane & 15) ^ (4 * t + (lane >> 4));
  }
  // Scales (wave 0): lanes 0..31 columns n0 + 4 l .. + 3 of the group of the
  // stage's first row, lanes 32..63 the same columns of the group of row 64.
  const int s_col = n0 + 4 * (lane & 31);
  const bool s_live = s_col < N;

  auto issue = [&](int ktl, int slot) {
    const int kt = kt0 + ktl;
    const int k0 = kt * kBK;
    lds_u8* base = (lds_u8*)smem + slot * kStage;
#pragma unroll
    for (int t = 0; t < 2; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xr, (__attribute__((address_space(3))) void*)(base + 1024 * (2 * wave + t)), 16,
          (a_off[t] >= 0 && k0 + 8 * swz(4 * (2 * wave + t) + (lane >> 4), lane & 15) < K)
              ? a_off[t] + 2 * k0 : kOutOfRange,
          0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int b = kt * 16 + b_sw[t];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          wr, (__attribute__((address_space(3))) void*)(base + kStageA + 1024 * (4 * wave + t)), 16,
          (b_live[t] && b < KB) ? b_off[t] + 16 * b : kOutOfRange, 0, 0, 0);
    }
    if (wave == 0) {
      const int g = (k0 + (lane >= 32 ? 64 : 0)) / G;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          sr, (__attribute__((address_space(3))) void*)(base + kStageA + kStageB), 16,
          s_live ? (g * N + s_col) * 4 : kOutOfRange, 0, 0, 0);
    }
  };

  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, each 16 rows x 64 columns
  const int fr = lane & 15, fq = lane >> 4;
  // LDS byte offsets (within a stage) of this lane's fragment reads, per k32
  // step h: X row wm 16 + l % 16; the piece 4 h + l / 16 of pair
  // 32 wn + 16 H + l % 16 (whose p % 16 is l % 16).
  int a_lds[4][1], b_lds[4][2];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
#pragma unroll
    for (int i = 0; i < 1; ++i) {
      const int row = wm * 16 + 16 * i + fr;
      a_lds[h][i] = row * kRowA + 16 * swz(row, 4 * h + fq);
    }
#pragma unroll
    for (int H = 0; H < 2; ++H)
      b_lds[h][H] = kStageA + (16 * (32 * wn + 16 * H + fr) + ((4 * h + fq) ^ fr)) * 16;
  }

  // acc: this group's sums of x * u (u = q + 128, as fp16 subnormals u 2^-24);
  // xacc: the same sums with every u = 128, i.e. 128 2^-24 sum(x), one
  // matrix-core product per row block against a constant operand; at the end
  // of a group tot += (acc - xacc) * scale, all in units of 2^-24.
  f32x4 acc[1][4], tot[1][4], xacc[1];
#pragma unroll
  for (int i = 0; i < 1; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  const h8 c128 = __builtin_bit_cast(h8, (u32x4){0x00800080u, 0x00800080u, 0x00800080u, 0x00800080u});

  // One k32 step of the stage in slot S: LDS reads; then each column's two
  // code bytes of a word into the low bytes of two fp16s whose other bits are
  // zero (the subnormals u 2^-24), one v_perm_b32 per register.
  struct Step {
    h8 a[1];
    u32x4 B[2];
  };
  auto read_step = [&](const unsigned char* S, int h, Step& st) {
#pragma unroll
    for (int i = 0; i < 1; ++i) st.a[i] = *reinterpret_cast<const h8*>(S + a_lds[h][i]);
#pragma unroll
    for (int H = 0; H < 2; ++H) st.B[H] = *reinterpret_cast<const u32x4*>(S + b_lds[h][H]);
  };
  auto convert = [&](const Step& st, h8 b[4]) {
#pragma unroll
    for (int H = 0; H < 2; ++H) {
      const u32x4 w = st.B[H];
      const u32x4 c0 = {q8_col_pair<0>(w[0]), q8_col_pair<0>(w[1]), q8_col_pair<0>(w[2]), q8_col_pair<0>(w[3])};
      const u32x4 c1 = {q8_col_pair<1>(w[0]), q8_col_pair<1>(w[1]), q8_col_pair<1>(w[2]), q8_col_pair<1>(w[3])};
      b[2 * H] = __builtin_bit_cast(h8, c0);
      b[2 * H + 1] = __builtin_bit_cast(h8, c1);
    }
  };
  auto group_end = [&](const unsigned char* S, int h) {
    // Scales of this lane's columns: v[H][0..1] for columns
    // 64 wn + 32 H + 8 (l / 16) + 0 .. 7 of the tile.
    const unsigned char* sc = S + kStageA + kStageB + 512 * (h >> 1) + 4 * (wn * 64 + 8 * fq);
    f32x4 v[2][2];
#pragma unroll
    for (int H = 0; H < 2; ++H)
#pragma unroll
      for (int e = 0; e < 2; ++e) v[H][e] = *reinterpret_cast<const f32x4*>(sc + 128 * H + 16 * e);
#pragma unroll
    for (int i = 0; i < 1; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int H = j >> 1, c = j & 1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 2 * r + c;  // column 8 (l / 16) + e of half H
          tot[i][j][r] = __builtin_fmaf(acc[i][j][r] - xacc[i][r], v[H][e >> 2][e & 3], tot[i][j][r]);
        }
      }
    }
  };
  // Software pipeline over the 4 k32 steps of a stage: step h + 1's LDS
  // reads are issued before step h's matrix-core work and its conversion
  // runs while those instructions execute.
  // gpos: offset of the stage's first row inside its group (a multiple of 64).
  auto compute = [&](int slot, int gpos) {
    const bool start0 = gpos == 0;          // a group starts at row 0 of the stage
    const bool mid = gpos + 64 == G;        // ... ends at row 63 and the next starts at 64
    const bool end3 = gpos + 128 == G || gpos + 128 == 2 * G;  // ... ends at row 127
    const unsigned char* S = smem + slot * kStage;
    Step st[2];
    h8 b[2][4];
    read_step(S, 0, st[0]);
    convert(st[0], b[0]);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (h < 3) read_step(S, h + 1, st[(h + 1) & 1]);
      // The first k32 step of a group starts its sums from zero.
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
      if ((h == 0 && start0) || (h == 2 && mid)) {
#pragma unroll
        for (int i = 0; i < 1; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[h & 1][j], st[h & 1].a[i], zero, 0, 0, 0);
          xacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(c128, st[h & 1].a[i], zero, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 1; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[h & 1][j], st[h & 1].a[i], acc[i][j], 0, 0, 0);
          xacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(c128, st[h & 1].a[i], xacc[i], 0, 0, 0);
        }
      }
      if (h < 3) convert(st[(h + 1) & 1], b[(h + 1) & 1]);
      if ((h == 1 && mid) || (h == 3 && end3)) group_end(S, h);
    }
  };

  issue(0, 0);
  if (nk > 1) issue(1, 1);
  int gpos = (kt0 * kBK) % G;  // 0: slices are whole groups
  for (int kt = 0; kt < nk; ++kt) {
    // Stage kt has landed for this wave (stage kt + 1 may be in flight).
    if (kt + 1 < nk) {
      if (wave == 0)
        wait_vmcnt<kLoads + 1>();
      else
        wait_vmcnt<kLoads>();
    } else {
      wait_vmcnt<0>();
    }
    // ... for every wave; and every wave is done with stage kt - 1, whose
    // slot takes stage kt + 2.
    lds_barrier();
    if (kt + 2 < nk) issue(kt + 2, (kt + 2) % kStages);
    compute(kt % kStages, gpos);
    gpos += kBK;
    gpos -= gpos >= G ? G : 0;
    gpos -= gpos >= G ? G : 0;
  }

#pragma unroll
  for (int i = 0; i < 1; ++i) {
    const int m = m0 + wm * 16 + 16 * i + fr;
    if (m >= M) continue;
#pragma unroll
    for (int H = 0; H < 2; ++H) {
      const int n = n0 + wn * 64 + 32 * H + 8 * fq;
      if (n >= N) continue;
      if (S > 1) {
        // Columns n + 2 r + c of tot[2 H + c][r]: 8 consecutive fp32.
        float* o = ws + ((size_t)slice * M + m) * N + n;
        const f32x4 lo = {tot[i][2 * H][0], tot[i][2 * H + 1][0], tot[i][2 * H][1], tot[i][2 * H + 1][1]};
        const f32x4 hi = {tot[i][2 * H][2], tot[i][2 * H + 1][2], tot[i][2 * H][3], tot[i][2 * H + 1][3]};
        *reinterpret_cast<f32x4*>(o) = lo;
        *reinterpret_cast<f32x4*>(o + 4) = hi;
        continue;
      }
      uint32_t w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const h2 pr = {(_Float16)(tot[i][2 * H][r] * kTwo24), (_Float16)(tot[i][2 * H + 1][r] * kTwo24)};
        w[r] = as_u32(pr);
      }
      *reinterpret_cast<uint4*>(Y + (size_t)m * N + n) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Y = fp16(2^24 * sum over the S slices, in slice order), 4 columns per thread.
__global__ __launch_bounds__(256) void q8_splitk_reduce_kernel(const float* __restrict__ ws,
                                                               _Float16* __restrict__ Y, int M,
                                                               int N, int S) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const size_t total = (size_t)M * N;
  if (i >= total) return;
  f32x4 a = *reinterpret_cast<const f32x4*>(ws + i);
  for (int sl = 1; sl < S; ++sl) a += *reinterpret_cast<const f32x4*>(ws + (size_t)sl * total + i);
  const h2 lo = {(_Float16)(a[0] * kTwo24), (_Float16)(a[1] * kTwo24)};
  const h2 hi = {(_Float16)(a[2] * kTwo24), (_Float16)(a[3] * kTwo24)};
  *reinterpret_cast<uint2*>(Y + i) = make_uint2(as_u32(lo), as_u32(hi));
}

bool q8_gemm_supported(int M, int K, int N, int G) {
  (void)M;
  (void)N;
  (void)K;
  return G % 64 == 0;
}

// K slices: enough workgroups to fill the GPU twice over (two fit on a CU),
// at most 8, each slice whole 128-row stages and whole groups.  The size of
// the workspace takes the largest S any group size allows (G <= 128).
static int q8_gemm_slices(int M, int K, int N, int G) {
  const int mtiles = (M + kBM - 1) / kBM, ntiles = (N + kBN - 1) / kBN;
  const int tiles = (ntiles + 7) / 8 * 8 * mtiles;
  const int unit = G > kBK ? G : kBK;  // rows per slice: a multiple of this
  int S = 1;
  while (S < 8 && tiles * 2 * S <= 2 * kTargetCUs && K % (unit * 2 * S) == 0) S *= 2;
  return S;
}
size_t q8_gemm_workspace_bytes(int M, int K, int N) {
  const int S = q8_gemm_slices(M, K, N, 64);
  return S > 1 ? (size_t)S * M * N * 4 : 0;
}

hipError_t launch_q8_gemm(const void* X, const void* packed, const float* scales, void* Y,
                          void* ws, int M, int K, int N, int G, hipStream_t s) {
  const int mtiles = (M + kBM - 1) / kBM, ntiles = (N + kBN - 1) / kBN;
  const int S = ws ? q8_gemm_slices(M, K, N, G) : 1;
  const int grid = (ntiles + 7) / 8 * 8 * mtiles * S;
  hipLaunchKernelGGL(q8_gemm_kernel, dim3(grid), dim3(kThreadsG), 0, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                     scales, reinterpret_cast<_Float16*>(Y), reinterpret_cast<float*>(ws), M, K, N,
                     G, K / 8, mtiles, ntiles, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const size_t quads = ((size_t)M * N) / 4;
  hipLaunchKernelGGL(q8_splitk_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<const float*>(ws), reinterpret_cast<_Float16*>(Y), M, N, S);
  return hipGetLastError();
}

}  // namespace wq
