// Internal launch interface between the C ABI (wq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace wq {

constexpr int kThreads = 256;  // 4 wave64s per workgroup

// Compute units the panel layouts are sized for (MI355X: 256).  Only the
// choice of panel width depends on it; launches use the device's own count.
constexpr int kTargetCUs = 256;

// Compute units of the current device (queried once per device).
int device_cus();

// Panel plan of a re-laid-out weight: a pure function of the shape, shared by
// the prepack kernel, the product and the unpack check.
//   P        panel width (columns); a panel spans all of K, and a workgroup
//            takes one panel or a contiguous run of them
//   cpp      column chunks per panel (16 columns for int8, 4 for 3/4-bit)
//   npanels  N / P
//   u        int8 / 3-bit: K units per slot (rows / 32-row blocks); slot s
//            covers units [s*u, s*u + u).  4-bit: 128-row blocks per panel
//   nsa      slots in use; threads in use = nsa * cpp
//   bw       unused (0)
//   threads  3-bit only: threads of the product's workgroup (slots = threads / cpp)
struct PanelPlan {
  int P, cpp, npanels, u, nsa, bw, threads;
  size_t packed_bytes;
};

PanelPlan plan_q8(int K, int N);
PanelPlan plan_q4(int K, int N, int G);
PanelPlan plan_q2(int K, int N, int G);
PanelPlan plan_q3(int K, int N);

hipError_t launch_q8_prepack(const int8_t* W, void* packed, int K, int N, hipStream_t s);
// ws: q8_group_workspace_bytes(M, K, N) bytes (unused when that is 0).
hipError_t launch_q8_group(const void* X, const void* packed, const float* scales, void* Y,
                           void* ws, int M, int K, int N, int G, hipStream_t s);
size_t q8_group_workspace_bytes(int M, int K, int N);
hipError_t launch_q8_unpack(const void* packed, int8_t* codes, int K, int N, hipStream_t s);
// Matrix-core path of the same product for more rows of X (q8_gemm.hip);
// with a workspace it splits K over workgroups (fp32 partial tiles in ws,
// summed in a fixed order by a second launch).
bool q8_gemm_supported(int M, int K, int N, int G);
size_t q8_gemm_workspace_bytes(int M, int K, int N);
hipError_t launch_q8_gemm(const void* X, const void* packed, const float* scales, void* Y,
                          void* ws, int M, int K, int N, int G, hipStream_t s);

// The separated form's dequantisation: W [K, N] = scale * q, fp32 or fp16.
hipError_t launch_q8_dequant(const int8_t* q, const float* scales, void* W, int K, int N, int G,
                             bool f16, hipStream_t s);

hipError_t launch_q3_prepack(const int32_t* qw, void* packed, int K, int N, hipStream_t s);
hipError_t launch_q3(const void* x, const void* packed, const void* scales, const void* zeros,
                     void* y, int K, int N, bool f16, hipStream_t s);
hipError_t launch_q3_unpack(const void* packed, int8_t* codes, int K, int N, hipStream_t s);

hipError_t launch_q4_prepack(const int32_t* qw, const int32_t* perm, void* packed, int K, int N,
                             int G, hipStream_t s);
// zeros: nullptr for the symmetric codes (offset 8), else fp16 [K/G, N].
// ws: q4_tiled_workspace_bytes(M, K) bytes (unused when that is 0).
hipError_t launch_q4_group(const void* X, const void* packed, const void* scales,
                           const void* zeros, void* Y, void* ws, int M, int K, int N, int G,
                           hipStream_t s);
// Byte offset, inside a 4-bit packed weight, of its forward row table
// (group-order row -> original row, 0xFFFF for padding rows).
size_t q4_fwd_table_offset(int K, int N);
// More than kQ4TiledMinRows rows of X: X is gathered into the packed
// weight's row order in the workspace (in matrix-core operand order, with
// the sums of X over runs of rows), then the tiled kernel reads the packed
// weight once per 64 rows (q4_tiled.hip).
constexpr int kQ4TiledMinRows = 4;
size_t q4_tiled_workspace_bytes(int M, int K);
hipError_t launch_q4_tiled(const void* X, const void* packed, const void* scales,
                           const void* zeros, void* Y, void* ws, int M, int K, int N, int G,
                           hipStream_t s);
hipError_t launch_q4_unpack(const void* packed, const int32_t* perm, int8_t* codes, int K, int N,
                            int G, hipStream_t s);
// 2-bit, asymmetric only (zeros required): the 4-bit kernel with 256-row blocks.
hipError_t launch_q2_prepack(const int32_t* qw, const int32_t* perm, void* packed, int K, int N,
                             int G, hipStream_t s);
hipError_t launch_q2_group(const void* X, const void* packed, const void* scales,
                           const void* zeros, void* Y, int M, int K, int N, int G, hipStream_t s);
hipError_t launch_q2_unpack(const void* packed, const int32_t* perm, int8_t* codes, int K, int N,
                            int G, hipStream_t s);

// Workspace of the W8A8 GEMM (and of the LLM.int8() decomposition) at this
// shape: the int32 partial tiles of its K slices, 0 when K is not split.
size_t w8a8_workspace_bytes(int M, int K, int N);
// The library's own W8A8 workspace (a device array of w8a8_scratch_bytes()
// bytes per GPU): its device address on the current device.
size_t w8a8_scratch_bytes();
hipError_t w8a8_scratch_ptr(void** out);
// smooth: nullptr, or the SmoothQuant factor s [K] (X is divided by it).
// ws: w8a8_workspace_bytes(M, K, N) bytes (unused when that is 0).
hipError_t launch_w8a8(const float* X, const float* smooth, const int8_t* Wq, const float* Sw,
                       void* Y, int8_t* Xq, float* Sx, int32_t* acc_out, void* ws, int M, int K,
                       int N, hipStream_t s);
// LLM.int8() decomposition: X16 [M, K] and W16 [N, K] fp16; Y [M, N] fp16;
// Xq, Sx, Wq, Sw (the quantised regular part), colmax [K], mask [K/32],
// out_cols [K] and n_out [1] are written.
hipError_t launch_int8_mixed(const void* X16, const void* W16, float threshold, void* Y,
                             int8_t* Xq, float* Sx, int8_t* Wq, float* Sw, float* colmax,
                             uint32_t* mask, int32_t* out_cols, int32_t* n_out, int32_t* acc_out,
                             void* ws, int M, int K, int N, hipStream_t s);

// Measurement references (calib.hip): a launch that does nothing, and one that
// only streams `bytes` of `buf` with the int8 GEMV's loads and grid shape.
hipError_t launch_calib_empty(int grid, int threads, uint32_t* sink, hipStream_t s);
hipError_t launch_calib_stream(const void* buf, int bytes, uint32_t* sink, hipStream_t s);

}  // namespace wq
