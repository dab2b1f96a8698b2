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
// Layout.  The [3K/32, N] weight is re-laid out once, offline
// (wq_prepack_q3), into column panels of P = 4*CPP columns over the whole of
// K.  Thread t = s*CPP + c takes the 4 columns of chunk c and the blocks of
// slot s; the three 16-byte word rows of one block of one chunk sit next to
// each other, and consecutive threads' blocks are consecutive, so the three
// loads of a step read 3 KB of contiguous memory per wave.  The activations
// are staged in LDS in the order the code pairs come out (q3_pair), each
// pair pre-scaled so that the subnormal code pairs of one accumulation class
// carry a common power of two.
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// fp16 activations: a pair is pre-scaled by 2^(cls - pa - kQ3XShift) and
// 2^(cls - pb - kQ3XShift), never by more than 1, so no finite fp16 x
// overflows (pre-scaling up by 2^(cls - p) alone would reach 4 x and turn
// |x| > 16376 into infinity); the 2^kQ3XShift returns in the final rescale.
constexpr int kQ3XShift = 2;
constexpr bool q3_prescale_at_most_one() {
  for (int P = 0; P < 16; ++P)
    if (q3_class(P) - q3_pair(P).pa > kQ3XShift || q3_class(P) - q3_pair(P).pb > kQ3XShift)
      return false;
  return true;
}
static_assert(q3_prescale_at_most_one(), "a pre-scale factor would exceed 1");

// Panels a workgroup walks at most: each keeps its waves' partial sums in
// its own LDS slot until the single reduction at the end.
constexpr int kQ3MaxRun = 8;

// Threads of the product's workgroup: 8 waves (two per SIMD, one wave's
// arithmetic overlapping another's loads) for the large shapes, 4 waves for
// the small ones, where the shorter per-wave staging wins, and a single wave
// when one wave's slots already cover K with one block each (the other waves
// would idle and still wait at the barrier).
static int q3_threads(int K, int N, int cpp) {
  if (K / 32 <= 64 / cpp && N <= 4096) return 64;
  return (K >= 8192 || N >= 8192) ? 512 : 256;
}

// Widest panel whose count spreads over kTargetCUs compute units in whole
// rounds with at most 12% idle (each workgroup then walks a contiguous run of
// panels); otherwise the narrowest width dividing N.
static int panel_width_3(int N) {
  int narrowest = 4;
  for (int P : {32, 16, 8, 4}) {
    if (N % P) continue;
    const int np = N / P, rounds = (np + kTargetCUs - 1) / kTargetCUs;
    if ((long long)rounds * kTargetCUs * 100 <= 112LL * np) return P;
    narrowest = P;
  }
  return narrowest;
}

PanelPlan plan_q3(int K, int N) {
  PanelPlan p{};
  p.P = panel_width_3(N);
  p.cpp = p.P / 4;
  p.npanels = N / p.P;
  p.threads = q3_threads(K, N, p.cpp);
  const int ns = p.threads / p.cpp;
  const int ku = K / 32;  // blocks
  p.u = (ku + ns - 1) / ns;
  p.nsa = (ku + p.u - 1) / p.u;
  p.packed_bytes = (size_t)p.npanels * p.u * p.nsa * p.cpp * 48;
  return p;
}

// ---------------------------------------------------------------------------
// Offline re-layout: one thread per (block, 4-column chunk) piece of 48 bytes.
// The piece's three 16-byte word rows are stored as three separate planes:
// word row j of piece (panel, i, t) sits at ((panel u + i) 3 + j) nta + t, so
// one load instruction of a wave (fixed i and j) reads 64 consecutive 16-byte
// words.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q3_prepack_kernel(const uint32_t* __restrict__ qw,
                                                              uint32_t* __restrict__ out, int K,
                                                              int N, PanelPlan p) {
  const int nta = p.nsa * p.cpp;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)p.npanels * p.u * nta;
  if (idx >= total) return;
  const int t = (int)(idx % nta);
  const size_t pi = idx / nta;
  const int i = (int)(pi % p.u), panel = (int)(pi / p.u);
  const int s = t / p.cpp, c = t % p.cpp;
  const int blk = s * p.u + i;
  const int col0 = panel * p.P + 4 * c;
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      out[((pi * 3 + j) * nta + t) * 4 + cc] = blk < K / 32 ? qw[(size_t)(3 * blk + j) * N + col0 + cc] : 0u;
}

// ---------------------------------------------------------------------------
// The fused product.
// ---------------------------------------------------------------------------
template <bool F16, int CPP, int THREADS>
__global__ __launch_bounds__(THREADS) void q3_panel_kernel(
    const void* __restrict__ xv, const uint8_t* __restrict__ Wp, const void* __restrict__ sv,
    const void* __restrict__ zv, void* __restrict__ yv, int K, int N, int u, int nsa, int pq,
    int pe, int packed_bytes) {
  constexpr int P = 4 * CPP;
  constexpr int LOWBIT = CPP == 1 ? 0 : CPP == 2 ? 1 : CPP == 4 ? 2 : 3;
  constexpr int NACC = F16 ? kQ3Classes : 1;
  constexpr int XW = F16 ? 1 : 2;  // LDS words per pair
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* xp = reinterpret_cast<uint32_t*>(smem);  // [K/2][XW]
  constexpr int UB = 1;  // 32-row blocks per streamed unit
  constexpr int NW = THREADS / 64;
  __shared__ float xsum_w[NW];
  __shared__ float red[kQ3MaxRun][NW][CPP][4];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // This workgroup's contiguous run of panels; a unit is UB blocks of a panel.
  const SplitPart part = split_part((int)blockIdx.x, pq, pe);
  const int p_begin = part.begin, p_end = part.begin + part.count;
  const int nr = (u + UB - 1) / UB;  // units per panel
  const int nunits = (p_end - p_begin) * nr;
  const int nta = nsa * CPP;
  const int c = t % CPP, s = t / CPP;
  const bool active = t < nta;
  const int ku = K / 32;
  const int blk0 = s * u;
  const int nblk = active ? (blk0 + u <= ku ? u : (ku > blk0 ? ku - blk0 : 0)) : 0;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, packed_bytes);
  // Load cursor (panel of the run, unit) walks the units in order; units past
  // the end of the run load nothing (out-of-range offsets).
  int lpi = 0, lu = 0;
  auto load_unit = [&](u32x4 (&w)[UB][3]) {
    const int panel = p_begin + lpi, i0 = lu * UB;
    const bool ok = panel < p_end;
#pragma unroll
    for (int i = 0; i < UB; ++i)
#pragma unroll
      for (int j = 0; j < 3; ++j)
        w[i][j] = buffer_stream(
            wr, (ok && i0 + i < nblk) ? ((((panel * u + i0 + i) * 3 + j) * nta + t) * 16) : kOutOfRange);
    if (++lu == nr) {
      lu = 0;
      ++lpi;
    }
  };

  // 1. Activations.  The slots of a wave cover a contiguous range of 32-row
  //    blocks, and a wave reads x only there, so each wave stages its own
  //    range into LDS and no workgroup barrier stands between the staging and
  //    the products.  All loads of the first XR rounds go out together, ahead
  //    of the weights.
  constexpr int XV = F16 ? 4 : 8;  // 16-byte loads per 32-row block of x
  constexpr int XR = 2;
  constexpr int SPW = 64 / CPP;    // slots per wave
  const int wlo = wave * SPW * u;
  const int whi = (wave + 1) * SPW * u < ku ? (wave + 1) * SPW * u : ku;
  const __amdgpu_buffer_rsrc_t xr_rsrc = make_rsrc(xv, K * (F16 ? 2 : 4));
  u32x4 xraw[XR][XV];
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int blk = wlo + lane + 64 * r;
#pragma unroll
    for (int v = 0; v < XV; ++v)
      xraw[r][v] = __builtin_amdgcn_raw_buffer_load_b128(
          xr_rsrc, blk < whi ? (blk * XV + v) * 16 : kOutOfRange, 0, 0);
  }

  // 2. The first two units of the weight stream.
  u32x4 w0[UB][3], w1[UB][3];
  load_unit(w0);
  load_unit(w1);

  // The scale and zero of output column p_begin * P + t (a run has at most
  // 32 * kQ3MaxRun <= THREADS outputs), loaded now and used at the end.
  // Issued after the first units, so waiting for those does not wait for them.
  // (launch_q3_t bounds the run so that a run's outputs never exceed THREADS.)
  const int nout = (p_end - p_begin) * P;
  float out_sc = 0.0f, out_ze = 0.0f;
  {
    // Buffer loads: they count in vmcnt only (a flat load would also hold up
    // every later LDS wait).
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sv, N * (F16 ? 2 : 4));
    const __amdgpu_buffer_rsrc_t zr = make_rsrc(zv, N * (F16 ? 2 : 4));
    const int off = t < nout ? (p_begin * P + t) * (F16 ? 2 : 4) : kOutOfRange;
    if constexpr (F16) {
      out_sc = (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0));
      out_ze = (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(zr, off, 0, 0));
    } else {
      out_sc = as_f32(__builtin_amdgcn_raw_buffer_load_b32(sr, off, 0, 0));
      out_ze = as_f32(__builtin_amdgcn_raw_buffer_load_b32(zr, off, 0, 0));
    }
  }

  // 3. Pairs into LDS in code-pair order (pre-scaled), and sum_k x[k].
  float my_sum = 0.0f;
  auto stage_block = [&](int blk, const u32x4* raw) {
    if constexpr (F16) {
      // The block's 32 halves sit in the 16 words raw[v][e] (word 4 v + e
      // holds rows 2 (4 v + e) and 2 (4 v + e) + 1).  sum_k x[k]: v_dot2
      // against ones.  Pair P: one v_perm_b32 takes row a's half into the
      // low and row b's half into the high half, and one packed fp16
      // multiply by the exact powers of two 2^(cls - pa - kQ3XShift),
      // 2^(cls - pb - kQ3XShift) (one rounding, as the fp32 ldexp and the
      // conversion to fp16 would give).
      const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) my_sum = dot2(as_h2(raw[v][e]), ones, my_sum);
      uint32_t pv[16];
#pragma unroll
      for (int P = 0; P < 16; ++P) {
        const Q3Pair q = q3_pair(P);
        const int cls = q3_class(P);
        const uint32_t wa = raw[q.a / 8][(q.a / 2) % 4], wb = raw[q.b / 8][(q.b / 2) % 4];
        // v_perm_b32(wb, wa, sel): selector bytes 0..3 pick wa's bytes,
        // 4..7 wb's.
        const uint32_t sel = (q.a & 1 ? 0x0302u : 0x0100u) | (q.b & 1 ? 0x07060000u : 0x05040000u);
        const h2 m = {(_Float16)__builtin_ldexpf(1.0f, cls - q.pa - kQ3XShift),
                      (_Float16)__builtin_ldexpf(1.0f, cls - q.pb - kQ3XShift)};
        pv[P] = as_u32(as_h2(__builtin_amdgcn_perm(wb, wa, sel)) * m);
      }
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        *reinterpret_cast<u32x4*>(xp + blk * 16 + 4 * v4) =
            u32x4{pv[4 * v4], pv[4 * v4 + 1], pv[4 * v4 + 2], pv[4 * v4 + 3]};
      return;
    }
    float xs[32];
#pragma unroll
    for (int v = 0; v < XV; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (F16) {
          const h2 hv = as_h2(raw[v][e]);
          xs[8 * v + 2 * e] = (float)hv.x;
          xs[8 * v + 2 * e + 1] = (float)hv.y;
        } else {
          xs[4 * v + e] = as_f32(raw[v][e]);
        }
      }
#pragma unroll
    for (int i = 0; i < 32; ++i) my_sum += xs[i];
#pragma unroll
    for (int P = 0; P < 16; ++P) {
      const Q3Pair q = q3_pair(P);
      if constexpr (F16) {
        // class = max(pa, pb): both products carry 2^(cls - 24 - kQ3XShift).
        const int cls = q3_class(P);
        const h2 hv = {(_Float16)__builtin_ldexpf(xs[q.a], cls - q.pa - kQ3XShift),
                       (_Float16)__builtin_ldexpf(xs[q.b], cls - q.pb - kQ3XShift)};
        xp[blk * 16 + P] = as_u32(hv);
      } else {
        // fp32: x as given; the code's 2^(p - 24) is undone on the code
        // itself (an exact power-of-two scale of a small integer), so no
        // finite x can overflow.
        xp[(blk * 16 + P) * 2] = __builtin_bit_cast(uint32_t, xs[q.a]);
        xp[(blk * 16 + P) * 2 + 1] = __builtin_bit_cast(uint32_t, xs[q.b]);
      }
    }
  };
#pragma unroll
  for (int r = 0; r < XR; ++r) {
    const int blk = wlo + lane + 64 * r;
    if (blk < whi) stage_block(blk, xraw[r]);
  }
  for (int blk = wlo + lane + 64 * XR; blk < whi; blk += 64) {
    u32x4 raw[XV];
#pragma unroll
    for (int v = 0; v < XV; ++v)
      raw[v] = __builtin_amdgcn_raw_buffer_load_b128(xr_rsrc, (blk * XV + v) * 16, 0, 0);
    stage_block(blk, raw);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) my_sum += __shfl_xor(my_sum, o);
  if (lane == 0) xsum_w[wave] = my_sum;  // read after the final barrier
  // The wave's own LDS writes are done before its lanes read each other's.
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");

  // 4. Exact codes times x, fp32 accumulation (one accumulator per class).
  float acc[NACC][4];
#pragma unroll
  for (int a = 0; a < NACC; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[a][j] = 0.0f;

  // One unit: multiply the buffer `w`, refill `pre` with unit q + 2; at the
  // last unit of a panel, reduce over the wave and leave the wave's partial
  // sums of the panel's P columns in LDS.
  int cpi = 0, cu = 0;  // compute cursor: panel of the run, unit
  auto step = [&](int q, const u32x4 (&w)[UB][3], u32x4 (&pre)[UB][3]) {
    if (q >= nunits) return;
    const int pr_i = cpi, i0 = cu * UB;
    const bool last = cu == nr - 1;
    if (++cu == nr) {
      cu = 0;
      ++cpi;
    }
#pragma unroll
    for (int i = 0; i < UB; ++i) {
      if (i0 + i >= nblk) break;
      const int blk = blk0 + i0 + i;
      uint32_t xr[16][XW];
      const u32x4* xq = reinterpret_cast<const u32x4*>(xp + (size_t)blk * 16 * XW);
#pragma unroll
      for (int v4 = 0; v4 < 4 * XW; ++v4) {
        const u32x4 tmp = xq[v4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xr[(v4 * 4 + e) / XW][(v4 * 4 + e) % XW] = tmp[e];
      }
#pragma unroll
      for (int col = 0; col < 4; ++col) {
        h2 pr[16];
        q3_block_pairs_sub(w[i][0][col], w[i][1][col], w[i][2][col], pr);
#pragma unroll
        for (int P = 0; P < 16; ++P) {
          if constexpr (F16) {
            const int slot = q3_class_slot(q3_class(P));
            acc[slot][col] = dot2(pr[P], as_h2(xr[P][0]), acc[slot][col]);
          } else {
            const float ua = (float)(1 << (24 - q3_pair(P).pa));
            const float ub = (float)(1 << (24 - q3_pair(P).pb));
            acc[0][col] = __builtin_fmaf((float)pr[P].x * ua, __builtin_bit_cast(float, xr[P][0]), acc[0][col]);
            acc[0][col] = __builtin_fmaf((float)pr[P].y * ub, __builtin_bit_cast(float, xr[P][1]), acc[0][col]);
          }
        }
      }
    }
    load_unit(pre);  // `w` is consumed: its registers take unit q + 2
    if (!last) return;

    // Classes back to one sum per column (powers of two: exact rescale).
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (F16) {
        float a = 0.0f;
#pragma unroll
        for (int sl = 0; sl < NACC; ++sl) {
          a = __builtin_fmaf(acc[sl][j], __builtin_ldexpf(1.0f, 24 + kQ3XShift - q3_slot_class(sl)), a);
          acc[sl][j] = 0.0f;
        }
        v[j] = a;
      } else {
        v[j] = acc[0][j];
        acc[0][j] = 0.0f;
      }
    }
    // Over the slots of a chunk that share this wave.
    bfly<4, 5, LOWBIT>(v, lane);
    bool owner;
    const int base = bfly_base<4, LOWBIT>(lane, owner);
    constexpr int LEFT = bfly_left<4, LOWBIT>();
    if (owner) {
#pragma unroll
      for (int j = 0; j < LEFT; ++j) red[pr_i][wave][c][base + j] = v[j];
    }
  };
  for (int q = 0; q < nunits; q += 2) {
    step(q, w0, w0);
    step(q + 1, w1, w1);
  }

  // 5. Over the waves, then y = scale * A - zero * sum(x), for every panel of
  //    the run at once.
  __syncthreads();
  float xsum = 0.0f;
#pragma unroll
  for (int w2 = 0; w2 < NW; ++w2) xsum += xsum_w[w2];
  if (t < nout) {
    const int pi = t / P, tt = t % P;
    const int rc = tt / 4, j = tt % 4;
    const int n = p_begin * P + t;
    float A = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) A += red[pi][w2][rc][j];
    if constexpr (F16)
      reinterpret_cast<_Float16*>(yv)[n] = (_Float16)(out_sc * A - out_ze * xsum);
    else
      reinterpret_cast<float*>(yv)[n] = out_sc * A - out_ze * xsum;
  }
}

// ---------------------------------------------------------------------------
// Bit-exact check: each packed block through q3_block_pairs_sub back to codes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q3_unpack_kernel(const uint8_t* __restrict__ Wp,
                                                             int8_t* __restrict__ codes, int K,
                                                             int N, PanelPlan p) {
  const int nta = p.nsa * p.cpp;
  const size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t total = (size_t)p.npanels * p.u * nta;
  if (idx >= total) return;
  const int t = (int)(idx % nta);
  const size_t pi = idx / nta;
  const int i = (int)(pi % p.u), panel = (int)(pi / p.u);
  const int s = t / p.cpp, c = t % p.cpp;
  const int blk = s * p.u + i;
  if (blk >= K / 32) return;
  const int col0 = panel * p.P + 4 * c;
  u32x4 w[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) w[j] = *reinterpret_cast<const u32x4*>(Wp + ((pi * 3 + j) * nta + t) * 16);
#pragma unroll
  for (int col = 0; col < 4; ++col) {
    h2 pr[16];
    q3_block_pairs_sub(w[0][col], w[1][col], w[2][col], pr);
#pragma unroll
    for (int P = 0; P < 16; ++P) {
      const uint32_t bits = as_u32(pr[P]);
      const int ca = (int)((bits & 0xFFFFu) >> q3_pair(P).pa);
      const int cb = (int)((bits >> 16) >> q3_pair(P).pb);
      codes[(size_t)(32 * blk + q3_pair(P).a) * N + col0 + col] = (int8_t)ca;
      codes[(size_t)(32 * blk + q3_pair(P).b) * N + col0 + col] = (int8_t)cb;
    }
  }
}

hipError_t launch_q3_prepack(const int32_t* qw, void* out, int K, int N, hipStream_t s) {
  const PanelPlan p = plan_q3(K, N);
  const size_t total = (size_t)p.npanels * p.u * p.nsa * p.cpp;
  hipLaunchKernelGGL(q3_prepack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(qw),
                     reinterpret_cast<uint32_t*>(out), K, N, p);
  return hipGetLastError();
}

hipError_t launch_q3_unpack(const void* packed, int8_t* codes, int K, int N, hipStream_t s) {
  const PanelPlan p = plan_q3(K, N);
  const size_t total = (size_t)p.npanels * p.u * p.nsa * p.cpp;
  hipLaunchKernelGGL(q3_unpack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint8_t*>(packed), codes, K, N, p);
  return hipGetLastError();
}

template <bool F16, int CPP, int THREADS>
static hipError_t launch_q3_t(const void* x, const void* packed, const void* scales,
                              const void* zeros, void* y, int K, int N, const PanelPlan& p,
                              hipStream_t s) {
  const size_t lds = (size_t)(K / 2) * (F16 ? 4 : 8);
  const int cus = device_cus();
  int grid = p.npanels < cus ? p.npanels : cus;
  // Runs of at most kQ3MaxRun panels and at most THREADS outputs (one per
  // thread in the final step).
  const int max_run = (THREADS / (4 * CPP)) < kQ3MaxRun ? THREADS / (4 * CPP) : kQ3MaxRun;
  if ((p.npanels + grid - 1) / grid > max_run) grid = (p.npanels + max_run - 1) / max_run;
  // Static LDS (the per-panel partial sums) plus x may pass 64 KB.
  constexpr size_t kStatic = sizeof(float) * ((size_t)kQ3MaxRun * (THREADS / 64) * CPP * 4 + THREADS / 64);
  if (lds + kStatic > 65536) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&q3_panel_kernel<F16, CPP, THREADS>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((q3_panel_kernel<F16, CPP, THREADS>), dim3(grid), dim3(THREADS), lds, s, x,
                     reinterpret_cast<const uint8_t*>(packed), scales, zeros, y, K, N, p.u, p.nsa,
                     p.npanels / grid, p.npanels % grid, (int)p.packed_bytes);
  return hipGetLastError();
}

// One 32-row block per unit: two units (six 16-byte loads a thread) stay in
// flight, which keeps the per-CU load queue busy without stalling the issue of
// the arithmetic behind a long run of loads.
template <bool F16, int CPP>
static hipError_t launch_q3_ub(const void* x, const void* packed, const void* scales,
                               const void* zeros, void* y, int K, int N, const PanelPlan& p,
                               hipStream_t s) {
  if (p.threads == 512) return launch_q3_t<F16, CPP, 512>(x, packed, scales, zeros, y, K, N, p, s);
  if (p.threads == 256) return launch_q3_t<F16, CPP, 256>(x, packed, scales, zeros, y, K, N, p, s);
  return launch_q3_t<F16, CPP, 64>(x, packed, scales, zeros, y, K, N, p, s);
}

template <bool F16>
static hipError_t launch_q3_f(const void* x, const void* packed, const void* scales,
                              const void* zeros, void* y, int K, int N, const PanelPlan& p,
                              hipStream_t s) {
  switch (p.cpp) {
    case 1: return launch_q3_ub<F16, 1>(x, packed, scales, zeros, y, K, N, p, s);
    case 2: return launch_q3_ub<F16, 2>(x, packed, scales, zeros, y, K, N, p, s);
    case 4: return launch_q3_ub<F16, 4>(x, packed, scales, zeros, y, K, N, p, s);
    default: return launch_q3_ub<F16, 8>(x, packed, scales, zeros, y, K, N, p, s);
  }
}

hipError_t launch_q3(const void* x, const void* packed, const void* scales, const void* zeros,
                     void* y, int K, int N, bool f16, hipStream_t s) {
  const PanelPlan p = plan_q3(K, N);
  return f16 ? launch_q3_f<true>(x, packed, scales, zeros, y, K, N, p, s)
             : launch_q3_f<false>(x, packed, scales, zeros, y, K, N, p, s);
}

}  // namespace wq
