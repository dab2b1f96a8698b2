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
// Tiles.  A workgroup owns a 64 x 128 tile of Y and walks K in stages of 64
// rows.  Per stage, direct-to-LDS buffer loads bring the X tile (fp16,
// 64 x 64), the int8 codes of the weight tile (64 rows x 128 columns, as the
// 16-byte pieces of the packed layout: one row of one 16-column chunk) and
// the stage's row of scales into a ring of kStages slots.  The codes of a
// stage are converted once per workgroup into an fp16 tile [n][k] (exact
// integers, via the fp16 magic number 1024 and one packed add), which the
// eight waves read as v_mfma_f32_16x16x32_f16 operands.  Each wave keeps a
// 32 x 32 accumulator for the current group and a running total; at the end
// of a group the total takes accumulator * scale (fp32) and the accumulator
// restarts, so the products are exact and every rounding is an fp32 one, as
// in the small-batch kernel.
//
// X rows and stage rows are 128-byte rows of 8 16-byte chunks; chunk c of
// row r sits at position c ^ ((r >> 1) & 7), which keeps the 16 rows of one
// fragment read on distinct LDS banks.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kBM = 64, kBN = 128, kBK = 64, kStages = 8, kThreadsG = 512;
constexpr int kRow = kBK * 2;                   // 128 bytes: one fp16 row of a stage
constexpr int kStageA = kBM * kRow;             // X tile, fp16 [m][k]
constexpr int kStageB = kBK * kBN;              // codes, 64 rows x 8 chunks of 16 bytes
constexpr int kStageS = 1024;                   // scales of the stage's group (512 bytes used)
constexpr int kStage = kStageA + kStageB + kStageS;
constexpr int kTileB = kBN * kRow;              // converted weight tile, fp16 [n][k]

__device__ __forceinline__ int swz(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// All LDS accesses of this wave done, then a workgroup barrier; the empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 8-byte LDS store issued as inline assembly.  A plain store into the same
// LDS array that the direct-to-LDS loads fill makes the compiler wait for
// every load in flight (it cannot tell the ring slots apart); here the
// ordering is explicit: the store follows the workgroup barrier that retires
// the tile's previous readers, and the barrier after the conversion waits for
// it (lgkmcnt(0)).
__device__ __forceinline__ void lds_store_b64(unsigned char* p, uint32_t lo, uint32_t hi) {
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_u8*)p;
  const uint64_t v = ((uint64_t)hi << 32) | lo;
  asm volatile("ds_write_b64 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Loads per stage per wave: X and codes; wave 0 also loads the scale row.
// Waiting until stage t + 1 has landed leaves the later stages in flight.
template <int PENDING_STAGES>
__device__ __forceinline__ void wait_stages(int wave) {
  if (wave == 0)
    wait_vmcnt<3 * PENDING_STAGES>();
  else
    wait_vmcnt<2 * PENDING_STAGES>();
}

}  // namespace

// Stage slot layout of the codes: piece (row r, chunk c) of a stage, r = 8 o
// + i, sits at 16-byte slot 8 (8 i + c) + o.  Load instruction i (one per
// wave) therefore brings row i of every octet o for all 8 chunks, and its 8
// lanes of one chunk read pieces that are consecutive in the packed layout
// whenever a slot of that layout holds 8 or more rows per chunk.
__global__ __launch_bounds__(kThreadsG) void q8_gemm_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const float* __restrict__ scales, _Float16* __restrict__ Y, int M, int K, int N, int G, int u,
    int nta, int cpp, int packed_bytes, int mtiles, int ntiles) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kStages * kStage + kTileB];
  unsigned char* const btile = smem + kStages * kStage;

  // Workgroups b and b + 8 run on the same XCD: the M tiles that share a
  // column tile of the weight are placed 8 apart.
  const int bid = blockIdx.x;
  const int grp = bid / (8 * mtiles), rr = bid % (8 * mtiles);
  const int mt = rr / 8, nt = grp * 8 + (rr % 8);
  if (nt >= ntiles) return;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nk = K / kBK;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(X, M * K * 2);
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, packed_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (K / G) * N * 4);

  // X: wave w loads stage rows 8w .. 8w + 7, lane l row 8w + l / 8, chunk
  // position l % 8.
  const int a_row = 8 * wave + (lane >> 3);
  const int a_off = m0 + a_row < M ? (m0 + a_row) * K * 2 + 16 * swz(a_row, lane & 7) : -1;
  // Codes: wave w loads row w of octet o = l % 8 of chunk l / 8.  The piece of
  // row k, chunk q sits at ((panel u + k % u) nta + (k / u) cpp + q % cpp) 16
  // with panel = q / cpp; (bs, bi) track (k / u, k % u) from stage to stage.
  const int q = n0 / 16 + (lane >> 3);
  const bool b_live = q < N / 16;
  const int b_panel = b_live ? q / cpp : 0, b_chunk = q % cpp;
  int bs, bi;
  {
    const int k = 8 * (lane & 7) + wave;
    bs = k / u;
    bi = k % u;
  }
  const int step_s = kBK / u, step_i = kBK % u;
  // Scales (wave 0): lane l < 32 loads columns n0 + 4 l .. + 3 of the group.
  const int s_col = n0 + 4 * lane;
  const bool s_live = lane < 32 && s_col < N;

  auto issue = [&](int kt, int slot) {
    const int k0 = kt * kBK;
    lds_u8* base = (lds_u8*)smem + slot * kStage;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(base + 1024 * wave), 16,
                                             a_off >= 0 ? a_off + 2 * k0 : kOutOfRange, 0, 0, 0);
    const int boff = ((b_panel * u + bi) * nta + bs * cpp + b_chunk) * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wr, (__attribute__((address_space(3))) void*)(base + kStageA + 1024 * wave), 16,
        b_live ? boff : kOutOfRange, 0, 0, 0);
    bi += step_i;
    const bool wrap = bi >= u;
    bi -= wrap ? u : 0;
    bs += step_s + (wrap ? 1 : 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          sr, (__attribute__((address_space(3))) void*)(base + kStageA + kStageB), 16,
          s_live ? ((k0 / G) * N + s_col) * 4 : kOutOfRange, 0, 0, 0);
  };

  // Codes of one stage -> fp16 tile [n][k].  Wave w takes rows 4 (w % 2) ..
  // + 3 of every octet of chunks 2 (w / 2) and 2 (w / 2) + 1; lane l: chunk
  // 2 (w / 2) + l / 32, octet (l / 4) % 8, 4-column group l % 4.  The 64
  // lanes of one read hit 64 distinct banks.
  const int cv_half = wave & 1, cv_chunk = 2 * (wave >> 1) + (lane >> 5);
  const int cv_oct = (lane >> 2) & 7, cv_grp = lane & 3;
  auto convert = [&](int slot) {
    const unsigned char* Bq = smem + slot * kStage + kStageA;
    unsigned char* Bt = btile;
    uint32_t D[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * cv_half + r;
      D[r] = *reinterpret_cast<const uint32_t*>(Bq + (8 * (8 * i + cv_chunk) + cv_oct) * 16 + 4 * cv_grp);
    }
    // Rows (0, 1) and (2, 3) interleaved per column: bytes c0r0 c0r1 c1r0 c1r1.
    const uint32_t t01[2] = {__builtin_amdgcn_perm(D[1], D[0], 0x05010400u),
                             __builtin_amdgcn_perm(D[1], D[0], 0x07030602u)};
    const uint32_t t23[2] = {__builtin_amdgcn_perm(D[3], D[2], 0x05010400u),
                             __builtin_amdgcn_perm(D[3], D[2], 0x07030602u)};
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // u = q + 128 into the low byte of fp16 1024 (0x64 high byte): 1024 + u.
      const uint32_t sel = (j & 1) ? 0x04030402u : 0x04010400u;
      const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, t01[j >> 1], sel)) + bias;
      const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, t23[j >> 1], sel)) + bias;
      const int n = 16 * cv_chunk + 4 * cv_grp + j;
      lds_store_b64(Bt + n * kRow + 16 * swz(n, cv_oct) + 8 * cv_half, as_u32(a), as_u32(b));
    }
  };

  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves, each 32 x 32
  const int fr = lane & 15, fq = lane >> 4;
  struct Frag {
    h8 a[2][2], b[2][2];
    f32x4 s[2];
  };
  auto read_frags = [&](int slot, bool group_end, Frag& f) {
    const unsigned char* As = smem + slot * kStage;
    const unsigned char* Bt = btile;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 4 * h + fq;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 32 + 16 * i + fr;
        f.a[h][i] = *reinterpret_cast<const h8*>(As + row * kRow + 16 * swz(row, c));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = wn * 32 + 16 * j + fr;
        f.b[h][j] = *reinterpret_cast<const h8*>(Bt + n * kRow + 16 * swz(n, c));
      }
    }
    if (group_end) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        f.s[j] = *reinterpret_cast<const f32x4*>(As + kStageA + kStageB +
                                                 4 * (wn * 32 + 16 * j + 4 * fq));
    }
  };

  // With the weight as the first operand the accumulator is C transposed:
  // lane l holds C[m][n .. n + 3], m = l % 16, n = 4 (l / 16).
  f32x4 acc[2][2], tot[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      tot[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    }
  auto mma = [&](const Frag& f, bool group_end) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(f.b[h][j], f.a[h][i], acc[i][j], 0, 0, 0);
    if (group_end) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r) tot[i][j][r] = __builtin_fmaf(acc[i][j][r], f.s[j][r], tot[i][j][r]);
          acc[i][j] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        }
    }
  };
  auto ends_group = [&](int kt) { return kt + 1 == nk || ((kt + 1) * kBK) % G == 0; };

  // Prologue: fill every slot, wait for stage 0, convert it, read it.
#pragma unroll
  for (int s = 0; s < kStages; ++s)
    if (s < nk) issue(s, s);
  if (nk >= kStages)
    wait_stages<kStages - 1>(wave);
  else
    wait_vmcnt<0>();
  lds_barrier();
  convert(0);
  lds_barrier();
  Frag F0, F1;
  read_frags(0, ends_group(0), F0);

  // Step t: stage t + 1 has landed for every wave; the slot of stage t (read
  // and converted already) is refilled with stage t + kStages; stage t + 1 is
  // converted and its fragments read; stage t (in registers) is multiplied.
  auto step = [&](int kt, Frag& cur, Frag& nxt) {
    if (kt + kStages - 1 < nk)
      wait_stages<kStages - 2>(wave);
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (kt + kStages < nk) issue(kt + kStages, kt % kStages);
    convert((kt + 1) % kStages);
    lds_barrier();
    read_frags((kt + 1) % kStages, ends_group(kt + 1), nxt);
    mma(cur, ends_group(kt));
  };
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    step(kt, F0, F1);
    step(kt + 1, F1, F0);
  }
  if (kt + 1 < nk) {
    step(kt, F0, F1);
    mma(F1, true);
  } else {
    mma(F0, true);
  }

#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 32 + 16 * i + fr;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 32 + 16 * j + 4 * fq;
      if (n >= N) continue;
      const h2 lo = {(_Float16)tot[i][j][0], (_Float16)tot[i][j][1]};
      const h2 hi = {(_Float16)tot[i][j][2], (_Float16)tot[i][j][3]};
      *reinterpret_cast<uint2*>(Y + (size_t)m * N + n) = make_uint2(as_u32(lo), as_u32(hi));
    }
  }
}

bool q8_gemm_supported(int M, int K, int N, int G) {
  (void)M;
  (void)N;
  return G % kBK == 0 && K % kBK == 0;
}

hipError_t launch_q8_gemm(const void* X, const void* packed, const float* scales, void* Y, int M,
                          int K, int N, int G, hipStream_t s) {
  const PanelPlan p = plan_q8(K, N);
  const int mtiles = (M + kBM - 1) / kBM, ntiles = (N + kBN - 1) / kBN;
  const int grid = (ntiles + 7) / 8 * 8 * mtiles;
  hipLaunchKernelGGL(q8_gemm_kernel, dim3(grid), dim3(kThreadsG), 0, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                     scales, reinterpret_cast<_Float16*>(Y), M, K, N, G, p.u, p.nsa * p.cpp, p.cpp,
                     (int)p.packed_bytes, mtiles, ntiles);
  return hipGetLastError();
}

}  // namespace wq
