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
// then into column panels over the whole of K in the order the threads read
// them.  At run time each workgroup scatters X into LDS through the inverse
// permutation (coalesced reads, LDS writes), so every 128-row batch a thread
// reads is one group, scaled once.
//
// Geometry.  A workgroup owns a panel of P = 4*CPP columns; thread
// t = s*CPP + c takes the 4 columns of chunk c (one 128-bit load per word
// row) and the u word rows of slot s, in batches of BW word rows (one group,
// or a part of one).  The activations sit in LDS as the pairs
// (rows 8r + j, 8r + j + 4) the codes come out in (q4_pairs_sub).
#include "wq_device.hpp"
#include "wq_internal.h"

namespace wq {

// Widest panel whose count spreads over kTargetCUs compute units in whole
// rounds with at most 12% idle (each workgroup then walks a contiguous run of
// panels); otherwise the narrowest width dividing N.
static int panel_width_4(int N) {
  int narrowest = 4;
  for (int P : {32, 16, 8, 4}) {
    if (N % P) continue;
    const int np = N / P, rounds = (np + kTargetCUs - 1) / kTargetCUs;
    if ((long long)rounds * kTargetCUs * 100 <= 112LL * np) return P;
    narrowest = P;
  }
  return narrowest;
}

PanelPlan plan_q4(int K, int N, int G) {
  PanelPlan p{};
  p.P = panel_width_4(N);
  p.cpp = p.P / 4;
  p.npanels = N / p.P;
  const int ns = kThreads / p.cpp;
  const int ku = K / 8;                       // word rows
  p.bw = (G / 8) < 16 ? (G / 8) : 16;         // word rows per batch: inside one group
  while (p.bw > 4 && ns * p.bw >= 2 * ku) p.bw /= 2;  // keep most slots busy
  p.u = p.bw * ((ku + ns * p.bw - 1) / (ns * p.bw));
  p.nsa = (ku + p.u - 1) / p.u;
  p.packed_bytes = (size_t)p.npanels * p.u * p.nsa * p.cpp * 16;
  return p;
}

// One LDS copy of X holds K rounded up to 64 rows (the swizzle below permutes
// word rows inside aligned groups of 8).
static inline int q4_kpad(int K) { return (K + 63) / 64 * 64; }

// Rows of X staged per launch: the LDS copies of X (MT * Kpad halves) stay
// <= 64 KB (plus the small cross-wave reduction buffer).
int q4_max_mt(int K) {
  int mt = 8;
  while (mt > 1 && (size_t)mt * q4_kpad(K) * 2 > 65536) mt /= 2;
  return mt;
}

// LDS word-row swizzle: slots that share a wave read different banks.  It
// only flips the low 3 bits of r, so it stays inside r's aligned 8-row group.
__device__ __forceinline__ int q4_swz(int r) { return r ^ ((r >> 4) & 7); }
// Half-word index of row i (in group order) inside one LDS copy of X.
__device__ __forceinline__ int q4_lds_half(int i) {
  const int r = i >> 3, j = i & 7;
  return (q4_swz(r) * 4 + (j & 3)) * 2 + (j >> 2);
}

// ---------------------------------------------------------------------------
// Offline re-layout: one thread per 16-byte piece (4 columns of a word row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q4_prepack_kernel(const uint32_t* __restrict__ qw,
                                                              const int* __restrict__ perm,
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
  const int r = s * p.u + i;  // word row in group order
  const int col0 = panel * p.P + 4 * c;
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    uint32_t word = 0;  // padding rows: u = 0, so they add nothing whatever x is
    if (r < K / 8) {
      word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int src = perm ? perm[8 * r + j] : 8 * r + j;
        const uint32_t sw = qw[(size_t)(src >> 3) * N + col0 + cc];
        word |= ((sw >> (4 * (src & 7))) & 15u) << (4 * j);
      }
    }
    out[idx * 4 + cc] = word;
  }
}

// ---------------------------------------------------------------------------
// The fused product.
// ---------------------------------------------------------------------------
template <int MT, int CPP, int BW>
__global__ __launch_bounds__(kThreads) void q4_panel_kernel(
    const _Float16* __restrict__ X, const uint8_t* __restrict__ Wp,
    const _Float16* __restrict__ scales, const int* __restrict__ invperm,
    _Float16* __restrict__ Y, int M, int K, int N, int G, int u, int nsa, int npanels,
    int packed_bytes) {
  constexpr int P = 4 * CPP;
  constexpr int V = 4 * MT;  // results per chunk: [m][4 columns]
  constexpr int LOWBIT = CPP == 1 ? 0 : CPP == 2 ? 1 : CPP == 4 ? 2 : 3;
  constexpr int LEFT = bfly_left<V, LOWBIT>();
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int kpad = (K + 63) / 64 * 64;  // halves per LDS copy of X
  _Float16* xh = reinterpret_cast<_Float16*>(smem);  // MT copies of kpad halves
  float* red = reinterpret_cast<float*>(smem + (size_t)MT * kpad * 2);  // [4 waves][CPP][V]

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // This workgroup's contiguous run of panels.
  const int p_begin = (int)((long long)blockIdx.x * npanels / gridDim.x);
  const int p_end = (int)((long long)(blockIdx.x + 1) * npanels / gridDim.x);
  const int nta = nsa * CPP;
  const int c = t % CPP, s = t / CPP;
  const bool active = t < nta;
  const int ku = K / 8;
  const int nb = u / BW;                        // batches per panel
  const int nunits = (p_end - p_begin) * nb;    // (panel, batch) units of the run

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(Wp, packed_bytes);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scales, (K / G) * N * 2);

  // A unit's loads: its scale pair first, then its BW weight pieces.  Units
  // past the end of the run load nothing (out-of-range offsets), so the loads
  // need no branch.
  u32x4 w0[BW], w1[BW], w2[BW];
  uint2 sc0, sc1, sc2;
  auto load_unit = [&](u32x4* dst, uint2& sc, int q) {
    const bool ok = active && q < nunits;
    const int panel = p_begin + q / nb, b = q % nb;
    const int r0 = s * u + b * BW;
    const int soff = (ok && r0 < ku) ? (((8 * r0) / G) * N + panel * P + 4 * c) * 2 : kOutOfRange;
    const unsigned long long v64 = __builtin_bit_cast(
        unsigned long long, __builtin_amdgcn_raw_buffer_load_b64(sr, soff, 0, 0));
    sc = make_uint2((uint32_t)v64, (uint32_t)(v64 >> 32));
    const int wbase = ((panel * u + b * BW) * nta + t) * 16;
#pragma unroll
    for (int i = 0; i < BW; ++i) dst[i] = buffer_stream(wr, ok ? wbase + i * nta * 16 : kOutOfRange);
  };

  // Scatter X into LDS through the inverse permutation (group order), once
  // for the whole run.  Thread t takes the 8-row chunks t, t + 256, ...; for
  // each chunk the permutation is read once and reused for every row of X.
  // All loads of a round of chunks go out before any LDS write; the first two
  // units of the weight stream go out right after the first round's loads.
  constexpr int CR = MT >= 8 ? 1 : 2;  // chunks per thread per round
  const int nchunk = K / 8;
  auto stage_load = [&](int c0, u32x4 (&pv)[CR][2], u32x4 (&xq)[CR][MT]) {
#pragma unroll
    for (int r = 0; r < CR; ++r) {
      const int ch = c0 + r * kThreads;
      const bool ok = ch < nchunk;
      if (invperm) {
        pv[r][0] = ok ? *reinterpret_cast<const u32x4*>(invperm + 8 * ch) : (u32x4){0u, 0u, 0u, 0u};
        pv[r][1] = ok ? *reinterpret_cast<const u32x4*>(invperm + 8 * ch + 4) : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
        xq[r][m] = (ok && m < M) ? *reinterpret_cast<const u32x4*>(X + (size_t)m * K + 8 * ch)
                                 : (u32x4){0u, 0u, 0u, 0u};
    }
  };
  auto stage_write = [&](int c0, const u32x4 (&pv)[CR][2], const u32x4 (&xq)[CR][MT]) {
#pragma unroll
    for (int r = 0; r < CR; ++r) {
      const int ch = c0 + r * kThreads;
      if (ch >= nchunk) break;
      int dst[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) dst[j] = invperm ? (int)pv[r][j >> 2][j & 3] : 8 * ch + j;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t word = xq[r][m][j >> 1];
          const uint16_t bits = (j & 1) ? (uint16_t)(word >> 16) : (uint16_t)(word & 0xFFFFu);
          reinterpret_cast<uint16_t*>(xh)[(size_t)m * kpad + q4_lds_half(dst[j])] = bits;
        }
    }
  };
  {
    u32x4 pv[CR][2], xq[CR][MT];
    stage_load(t, pv, xq);
    load_unit(w0, sc0, 0);
    load_unit(w1, sc1, 1);
    stage_write(t, pv, xq);
  }
  for (int c0 = t + CR * kThreads; c0 < nchunk; c0 += CR * kThreads) {
    u32x4 pv[CR][2], xq[CR][MT];
    stage_load(c0, pv, xq);
    stage_write(c0, pv, xq);
  }
  __syncthreads();

  const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  float accT[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) accT[m][j] = 0.0f;

  // Units go through a ring of three register buffers: while unit q is
  // multiplied, units q + 1 and q + 2 are in flight.  The loop is unrolled by
  // three so every buffer keeps a fixed set of registers (a register copy of
  // a buffer would wait for its loads).
  auto step = [&](int q, const u32x4* w, const uint2& sraw, u32x4* pre, uint2& pre_sc) {
    load_unit(pre, pre_sc, q + 2);
    if (q >= nunits) return;
    const int panel = p_begin + q / nb, b = q % nb;
    const int r0 = s * u + b * BW;  // first word row of the batch (group order)
    // Sum of x over the batch: the CPP lanes of a slot split the word rows.
    float xs[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) xs[m] = 0.0f;
    for (int i = c; i < BW; i += CPP) {
      const int r = r0 + i;
      if (r < ku) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xh + (size_t)m * kpad + q4_swz(r) * 8);
#pragma unroll
          for (int j = 0; j < 4; ++j) xs[m] = dot2(as_h2(xv[j]), ones, xs[m]);
        }
      }
    }
#pragma unroll
    for (int o = 1; o < CPP; o <<= 1)
#pragma unroll
      for (int m = 0; m < MT; ++m) xs[m] += __shfl_xor(xs[m], o);

    // Codes are u = q + 8: start at -8 * sum(x) (2^-24 units).  acc0 holds the
    // even nibbles (u * 2^-24), acc4 the odd ones (16u * 2^-24).
    float acc0[MT][4], acc4[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0[m][j] = xs[m] * (-8.0f / kTwo24);
        acc4[m][j] = 0.0f;
      }
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      const int r = r0 + i < ku ? r0 + i : ku - 1;  // rows past K: codes are 0, any x
      u32x4 xv[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) xv[m] = *reinterpret_cast<const u32x4*>(xh + (size_t)m * kpad + q4_swz(r) * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h2 pr[4];
        q4_pairs_sub(w[i][j], pr);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc0[m][j] = dot2(pr[0], as_h2(xv[m][0]), acc0[m][j]);
          acc4[m][j] = dot2(pr[1], as_h2(xv[m][1]), acc4[m][j]);
          acc0[m][j] = dot2(pr[2], as_h2(xv[m][2]), acc0[m][j]);
          acc4[m][j] = dot2(pr[3], as_h2(xv[m][3]), acc4[m][j]);
        }
      }
    }
    const h2 s01 = as_h2(sraw.x), s23 = as_h2(sraw.y);
    const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        accT[m][j] = __builtin_fmaf(__builtin_fmaf(acc4[m][j], 0.0625f, acc0[m][j]), sc[j], accT[m][j]);

    if (b == nb - 1) {
      // Panel done: reduce over the slots of each chunk and write P x MT results.
      float v[V];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[m * 4 + j] = accT[m][j];
          accT[m][j] = 0.0f;
        }
      bfly<V, 5, LOWBIT>(v, lane);
      bool owner;
      const int base = bfly_base<V, LOWBIT>(lane, owner);
      if (owner) {
#pragma unroll
        for (int j = 0; j < LEFT; ++j) red[(wave * CPP + c) * V + base + j] = v[j];
      }
      __syncthreads();
      for (int r = t; r < CPP * V; r += kThreads) {
        const int rc = r / V, idx = r % V;
        const int m = idx / 4, col = panel * P + 4 * rc + (idx % 4);
        float sum = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < kThreads / 64; ++w2) sum += red[(w2 * CPP + rc) * V + idx];
        if (m < M) Y[(size_t)m * N + col] = (_Float16)(sum * kTwo24);
      }
      __syncthreads();  // red is rewritten by the next panel
    }
  };
  for (int q = 0; q < nunits; q += 3) {
    step(q, w0, sc0, w2, sc2);
    step(q + 1, w1, sc1, w0, sc0);
    step(q + 2, w2, sc2, w1, sc1);
  }
}

// ---------------------------------------------------------------------------
// Bit-exact check: packed pieces through q4_pairs_sub back to signed codes in
// the original row order (perm), one thread per piece.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void q4_unpack_kernel(const uint8_t* __restrict__ Wp,
                                                             const int* __restrict__ perm,
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
  const int r = s * p.u + i;
  if (r >= K / 8) return;
  const int col0 = panel * p.P + 4 * c;
  const u32x4 w = *reinterpret_cast<const u32x4*>(Wp + idx * 16);
#pragma unroll
  for (int cc = 0; cc < 4; ++cc) {
    h2 pr[4];
    q4_pairs_sub(w[cc], pr);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t bits = as_u32(pr[j]);
      const int sh = (j & 1) ? 4 : 0;  // pairs 1 and 3 sit at bit 4 of each half
      const int ulo = (int)((bits & 0xFFFFu) >> sh), uhi = (int)((bits >> 16) >> sh);
      const int ia = 8 * r + j, ib = ia + 4;
      const int da = perm ? perm[ia] : ia, db = perm ? perm[ib] : ib;
      codes[(size_t)da * N + col0 + cc] = (int8_t)(ulo - 8);
      codes[(size_t)db * N + col0 + cc] = (int8_t)(uhi - 8);
    }
  }
}

hipError_t launch_q4_prepack(const int32_t* qw, const int32_t* perm, void* out, int K, int N, int G,
                             hipStream_t s) {
  const PanelPlan p = plan_q4(K, N, G);
  const size_t total = (size_t)p.npanels * p.u * p.nsa * p.cpp;
  hipLaunchKernelGGL(q4_prepack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint32_t*>(qw), perm,
                     reinterpret_cast<uint32_t*>(out), K, N, p);
  return hipGetLastError();
}

hipError_t launch_q4_unpack(const void* packed, const int32_t* perm, int8_t* codes, int K, int N,
                            int G, hipStream_t s) {
  const PanelPlan p = plan_q4(K, N, G);
  const size_t total = (size_t)p.npanels * p.u * p.nsa * p.cpp;
  hipLaunchKernelGGL(q4_unpack_kernel, dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, s, reinterpret_cast<const uint8_t*>(packed), perm, codes, K,
                     N, p);
  return hipGetLastError();
}

template <int MT, int CPP, int BW>
static hipError_t launch_q4_t(const void* X, const void* packed, const void* scales,
                              const int32_t* invperm, void* Y, int M, int K, int N, int G,
                              const PanelPlan& p, hipStream_t s) {
  const size_t xb = (size_t)MT * q4_kpad(K) * 2, rb = (size_t)kThreads / 64 * CPP * 4 * MT * 4;
  const int cus = device_cus();
  const int grid = p.npanels < cus ? p.npanels : cus;
  if (xb + rb > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&q4_panel_kernel<MT, CPP, BW>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(xb + rb));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((q4_panel_kernel<MT, CPP, BW>), dim3(grid), dim3(kThreads), xb + rb, s,
                     reinterpret_cast<const _Float16*>(X), reinterpret_cast<const uint8_t*>(packed),
                     reinterpret_cast<const _Float16*>(scales), invperm,
                     reinterpret_cast<_Float16*>(Y), M, K, N, G, p.u, p.nsa, p.npanels,
                     (int)p.packed_bytes);
  return hipGetLastError();
}

// Batch size: the plan's (one group, at most 16 word rows), smaller for
// larger MT to stay inside the register file.  Any power of two up to the
// plan's batch divides u, so the packed layout does not depend on it.
template <int MT, int CPP>
static hipError_t launch_q4_bw(const void* X, const void* packed, const void* scales,
                               const int32_t* invperm, void* Y, int M, int K, int N, int G,
                               const PanelPlan& p, hipStream_t s) {
  constexpr int cap = MT >= 8 ? 4 : (MT >= 4 ? 8 : 16);
  const int bw = p.bw < cap ? p.bw : cap;
  switch (bw) {
    case 4: return launch_q4_t<MT, CPP, 4>(X, packed, scales, invperm, Y, M, K, N, G, p, s);
    case 8: return launch_q4_t<MT, CPP, (cap < 8 ? 4 : 8)>(X, packed, scales, invperm, Y, M, K, N, G, p, s);
    default: return launch_q4_t<MT, CPP, cap>(X, packed, scales, invperm, Y, M, K, N, G, p, s);
  }
}

template <int MT>
static hipError_t launch_q4_mt(const void* X, const void* packed, const void* scales,
                               const int32_t* invperm, void* Y, int M, int K, int N, int G,
                               const PanelPlan& p, hipStream_t s) {
  switch (p.cpp) {
    case 1: return launch_q4_bw<MT, 1>(X, packed, scales, invperm, Y, M, K, N, G, p, s);
    case 2: return launch_q4_bw<MT, 2>(X, packed, scales, invperm, Y, M, K, N, G, p, s);
    case 4: return launch_q4_bw<MT, 4>(X, packed, scales, invperm, Y, M, K, N, G, p, s);
    default: return launch_q4_bw<MT, 8>(X, packed, scales, invperm, Y, M, K, N, G, p, s);
  }
}

hipError_t launch_q4_group(const void* X, const void* packed, const void* scales,
                           const int32_t* invperm, void* Y, int M, int K, int N, int G,
                           hipStream_t s) {
  const PanelPlan p = plan_q4(K, N, G);
  const int mtmax = q4_max_mt(K);
  for (int m0 = 0; m0 < M; m0 += mtmax) {
    const int mc = (M - m0) < mtmax ? (M - m0) : mtmax;
    const int mt = mc == 1 ? 1 : (mc == 2 ? 2 : (mc <= 4 ? 4 : 8));
    const void* Xc = reinterpret_cast<const char*>(X) + (size_t)m0 * K * 2;
    void* Yc = reinterpret_cast<char*>(Y) + (size_t)m0 * N * 2;
    hipError_t e;
    switch (mt) {
      case 1: e = launch_q4_mt<1>(Xc, packed, scales, invperm, Yc, mc, K, N, G, p, s); break;
      case 2: e = launch_q4_mt<2>(Xc, packed, scales, invperm, Yc, mc, K, N, G, p, s); break;
      case 4: e = launch_q4_mt<4>(Xc, packed, scales, invperm, Yc, mc, K, N, G, p, s); break;
      default: e = launch_q4_mt<8>(Xc, packed, scales, invperm, Yc, mc, K, N, G, p, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace wq
