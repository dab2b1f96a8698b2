// Internal launch interface between the C ABI (wq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

// Workgroup geometry shared by the weight-only kernels: 256 threads
// (4 wave64s) cover a 256-column tile; K is split over `splits` workgroups.
constexpr int kThreads = 256;
constexpr int kTileN = 256;

struct SplitPlan {
  int n_tiles;   // column tiles
  int splits;    // workgroups per column tile along K (S)
  int unit;      // kernel-specific tiling parameter (rows per lane span, ...)
  int mt;        // rows of X handled per launch (weight-only GEMM)
};

// Workspace layout: [counters: n_tiles uint32, padded to 256 B][partials: S*mt*N fp32]
inline size_t ws_counter_bytes(int n_tiles) { return ((size_t)n_tiles * 4 + 255) / 256 * 256; }
inline size_t ws_bytes(const SplitPlan& p, int N) {
  if (p.splits <= 1) return ws_counter_bytes(p.n_tiles);
  return ws_counter_bytes(p.n_tiles) + (size_t)p.splits * p.mt * N * 4;
}

SplitPlan plan_q8(int M, int K, int N, int G);
SplitPlan plan_q3(int K, int N);
SplitPlan plan_q4(int M, int K, int N, int G);

hipError_t launch_q8_group(const void* X, const int8_t* Wq, const float* scales, void* Y,
                           int M, int K, int N, int G, const SplitPlan& p, void* ws,
                           hipStream_t s);
hipError_t launch_q3(const void* x, const int32_t* qw, const void* scales, const void* zeros,
                     void* y, int K, int N, bool f16, const SplitPlan& p, void* ws,
                     hipStream_t s);
hipError_t launch_q4_group(const void* X, const int32_t* qw, const void* scales,
                           const int32_t* perm, void* Y, int M, int K, int N, int G,
                           const SplitPlan& p, void* ws, hipStream_t s);
hipError_t launch_q4_prepack(const int32_t* qw, const int32_t* perm, int32_t* out, int K, int N,
                             hipStream_t s);
hipError_t launch_unpack_q3(const int32_t* qw, int8_t* codes, int K, int N, hipStream_t s);
hipError_t launch_unpack_q4(const int32_t* qw, const int32_t* perm, int8_t* codes, int K, int N,
                            hipStream_t s);
hipError_t launch_w8a8(const float* X, const int8_t* Wq, const float* Sw, void* Y, int8_t* Xq,
                       float* Sx, int32_t* acc_out, int M, int K, int N, hipStream_t s);

// Tuning override for sweeps: WQ_SPLITK_UNIT=<n> replaces the kernel's
// tiling parameter when it is a supported value (0 = not set).
int env_unit_override();

}  // namespace wq
