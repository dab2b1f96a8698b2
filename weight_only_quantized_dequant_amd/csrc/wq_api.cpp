// C ABI of libwq.so: argument checks (all before any HIP call) and launches.
// Declarations and contracts: include/wq.h.
#include "../../include/wq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <vector>

#include "wq_internal.h"

namespace wq {

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kTargetCUs;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = kTargetCUs;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace wq

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return WQ_OK;
  g_last_hip_error = (int)e;
  return WQ_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Byte extents addressed through 32-bit buffer offsets.
constexpr long long kMaxBytes = 0x7FFFFFF0LL;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_q3(int K, int N) {
  if (K < 32 || N < 4 || K % 32 || N % 4) return WQ_ERR_SHAPE;
  if ((long long)(K / 32) * 3 * N * 4 > kMaxBytes / 2) return WQ_ERR_SHAPE;
  return WQ_OK;
}

int check_q8(int K, int N) {
  if (K < 32 || N < 16 || K % 32 || N % 16) return WQ_ERR_SHAPE;
  if ((long long)K * N > kMaxBytes / 2) return WQ_ERR_SHAPE;
  return WQ_OK;
}

int check_q4(int K, int N, int G) {
  if (G < 32 || !pow2(G) || K < G || K % G || N < 4 || N % 4) return WQ_ERR_SHAPE;
  if (K > 32768) return WQ_ERR_SHAPE;  // X staged in LDS; 16-bit row table
  if ((long long)(K / 8) * N * 4 > kMaxBytes / 2) return WQ_ERR_SHAPE;
  return WQ_OK;
}

// 2-bit: the 4-bit limits; the packed weight is a quarter of K*N bytes.
int check_q2(int K, int N, int G) {
  if (G < 32 || !pow2(G) || K < G || K % G || N < 4 || N % 4) return WQ_ERR_SHAPE;
  if (K > 32768) return WQ_ERR_SHAPE;  // X staged in LDS; 16-bit row table
  if ((long long)(K / 16) * N * 4 > kMaxBytes / 2) return WQ_ERR_SHAPE;
  return WQ_OK;
}

}  // namespace

extern "C" {

size_t wq_packed_bytes(int op, int K, int N, int G) {
  switch (op) {
    case WQ_OP_Q3: return check_q3(K, N) ? 0 : wq::plan_q3(K, N).packed_bytes;
    case WQ_OP_Q4G: return check_q4(K, N, G) ? 0 : wq::plan_q4(K, N, G).packed_bytes;
    case WQ_OP_Q8G: return check_q8(K, N) ? 0 : wq::plan_q8(K, N).packed_bytes;
    case WQ_OP_Q2G: return check_q2(K, N, G) ? 0 : wq::plan_q2(K, N, G).packed_bytes;
    default: return 0;
  }
}

// ------------------------------------------------------------------ 3-bit --

int wq_prepack_q3(const int32_t* qweight, void* packed, int K, int N, void* stream) {
  if (!qweight || !packed) return WQ_ERR_NULL;
  if (int st = check_q3(K, N)) return st;
  if (!aligned16(qweight) || !aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q3_prepack(qweight, packed, K, N, as_stream(stream)));
}

int wq_matvec_q3(const void* x, const void* packed, const void* scales, const void* zeros,
                 void* y, int K, int N, int dtype, void* stream) {
  if (!x || !packed || !scales || !zeros || !y) return WQ_ERR_NULL;
  if (dtype != WQ_F32 && dtype != WQ_F16) return WQ_ERR_DTYPE;
  if (int st = check_q3(K, N)) return st;
  if (K > (dtype == WQ_F16 ? 32768 : 16384)) return WQ_ERR_SHAPE;  // x staged in 64 KB of LDS
  if (!aligned16(x) || !aligned16(packed) || !aligned16(scales)) return WQ_ERR_ALIGN;
  return hip_status(
      wq::launch_q3(x, packed, scales, zeros, y, K, N, dtype == WQ_F16, as_stream(stream)));
}

int wq_unpack_q3(const void* packed, int8_t* codes, int K, int N, void* stream) {
  if (!packed || !codes) return WQ_ERR_NULL;
  if (int st = check_q3(K, N)) return st;
  if (!aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q3_unpack(packed, codes, K, N, as_stream(stream)));
}

// ------------------------------------------------------------------- int8 --

int wq_prepack_q8(const int8_t* qweight, void* packed, int K, int N, void* stream) {
  if (!qweight || !packed) return WQ_ERR_NULL;
  if (int st = check_q8(K, N)) return st;
  if (!aligned16(qweight) || !aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q8_prepack(qweight, packed, K, N, as_stream(stream)));
}

int wq_gemm_q8_group(const void* X, const void* packed, const float* scales, void* Y, int M,
                     int K, int N, int G, void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !packed || !scales || !Y) return WQ_ERR_NULL;
  if (int st = check_q8(K, N)) return st;
  if (M < 1 || G < 32 || G % 32 || K % G) return WQ_ERR_SHAPE;
  if ((long long)M * K * 2 > kMaxBytes || (long long)(K / G) * N * 4 > kMaxBytes)
    return WQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(scales) || !aligned16(Y))
    return WQ_ERR_ALIGN;
  // The tiled path (groups of 64 rows or more) splits K through the
  // workspace when its tiles alone do not fill the GPU.
  const size_t need = G % 64 == 0 ? wq::q8_group_workspace_bytes(M, K, N) : 0;
  if (need > (size_t)kMaxBytes) return WQ_ERR_SHAPE;
  if (need && (!workspace || workspace_bytes < need)) return WQ_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q8_group(X, packed, scales, Y, need ? workspace : nullptr, M, K, N,
                                        G, as_stream(stream)));
}

int wq_dequant_q8_group(const int8_t* qweight, const float* scales, void* W, int K, int N, int G,
                        int dtype, void* stream) {
  if (!qweight || !scales || !W) return WQ_ERR_NULL;
  if (int st = check_q8(K, N)) return st;
  if (G < 32 || G % 32 || K % G || (dtype != WQ_F32 && dtype != WQ_F16)) return WQ_ERR_SHAPE;
  if ((long long)K * N * (dtype == WQ_F32 ? 4 : 2) > kMaxBytes) return WQ_ERR_SHAPE;
  if (!aligned16(qweight) || !aligned16(scales) || !aligned16(W)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q8_dequant(qweight, scales, W, K, N, G, dtype == WQ_F16,
                                          as_stream(stream)));
}

int wq_unpack_q8(const void* packed, int8_t* codes, int K, int N, void* stream) {
  if (!packed || !codes) return WQ_ERR_NULL;
  if (int st = check_q8(K, N)) return st;
  if (!aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q8_unpack(packed, codes, K, N, as_stream(stream)));
}

// ------------------------------------------------------------------ 4-bit --

int wq_q4_act_order_perm(const int32_t* g_idx, int K, int G, int32_t* perm, int32_t* invperm) {
  if (!perm || !invperm) return WQ_ERR_NULL;
  if (K < 1 || G < 1 || K % G) return WQ_ERR_SHAPE;
  const int ng = K / G;
  if (!g_idx) {
    for (int k = 0; k < K; ++k) perm[k] = invperm[k] = k;
    return WQ_OK;
  }
  std::vector<int> count(ng, 0);
  for (int k = 0; k < K; ++k) {
    const int g = g_idx[k];
    if (g < 0 || g >= ng) return WQ_ERR_SHAPE;
    ++count[g];
  }
  for (int g = 0; g < ng; ++g)
    if (count[g] != G) return WQ_ERR_SHAPE;
  std::vector<int> next(ng);
  for (int g = 0; g < ng; ++g) next[g] = g * G;
  for (int k = 0; k < K; ++k) {  // stable within a group
    const int i = next[g_idx[k]]++;
    perm[i] = k;
    invperm[k] = i;
  }
  return WQ_OK;
}

int wq_prepack_q4(const int32_t* qweight, const int32_t* perm, void* packed, int K, int N, int G,
                  void* stream) {
  if (!qweight || !packed) return WQ_ERR_NULL;
  if (int st = check_q4(K, N, G)) return st;
  if (!aligned16(qweight) || !aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q4_prepack(qweight, perm, packed, K, N, G, as_stream(stream)));
}

namespace {

// The 4-bit products above kQ4TiledMinRows rows take a workspace for X in
// the packed weight's row order (read through 32-bit buffer offsets).
int check_q4_ws(int M, int K, const void* ws, size_t ws_bytes) {
  const size_t need = wq::q4_tiled_workspace_bytes(M, K);
  if (need == 0) return WQ_OK;
  if (need > (size_t)kMaxBytes) return WQ_ERR_SHAPE;
  if (!ws || ws_bytes < need) return WQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return WQ_ERR_ALIGN;
  return WQ_OK;
}

}  // namespace

int wq_gemm_q4_group(const void* X, const void* packed, const void* scales, void* Y, int M, int K,
                     int N, int G, void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !packed || !scales || !Y) return WQ_ERR_NULL;
  if (int st = check_q4(K, N, G)) return st;
  if (M < 1) return WQ_ERR_SHAPE;
  if ((long long)M * K * 2 > kMaxBytes) return WQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(scales)) return WQ_ERR_ALIGN;
  if (int st = check_q4_ws(M, K, workspace, workspace_bytes)) return st;
  return hip_status(wq::launch_q4_group(X, packed, scales, nullptr, Y, workspace, M, K, N, G,
                                        as_stream(stream)));
}

int wq_gemm_q4_group_zp(const void* X, const void* packed, const void* scales, const void* zeros,
                        void* Y, int M, int K, int N, int G, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!X || !packed || !scales || !zeros || !Y) return WQ_ERR_NULL;
  if (int st = check_q4(K, N, G)) return st;
  if (M < 1) return WQ_ERR_SHAPE;
  if ((long long)M * K * 2 > kMaxBytes) return WQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(scales) || !aligned16(zeros))
    return WQ_ERR_ALIGN;
  if (int st = check_q4_ws(M, K, workspace, workspace_bytes)) return st;
  return hip_status(wq::launch_q4_group(X, packed, scales, zeros, Y, workspace, M, K, N, G,
                                        as_stream(stream)));
}

int wq_unpack_q4(const void* packed, const int32_t* perm, int8_t* codes, int K, int N, int G,
                 void* stream) {
  if (!packed || !codes) return WQ_ERR_NULL;
  if (int st = check_q4(K, N, G)) return st;
  if (!aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q4_unpack(packed, perm, codes, K, N, G, as_stream(stream)));
}

// ------------------------------------------------------------------ 2-bit --

int wq_prepack_q2(const int32_t* qweight, const int32_t* perm, void* packed, int K, int N, int G,
                  void* stream) {
  if (!qweight || !packed) return WQ_ERR_NULL;
  if (int st = check_q2(K, N, G)) return st;
  if (!aligned16(qweight) || !aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q2_prepack(qweight, perm, packed, K, N, G, as_stream(stream)));
}

int wq_gemm_q2_group_zp(const void* X, const void* packed, const void* scales, const void* zeros,
                        void* Y, int M, int K, int N, int G, void* stream) {
  if (!X || !packed || !scales || !zeros || !Y) return WQ_ERR_NULL;
  if (int st = check_q2(K, N, G)) return st;
  if (M < 1) return WQ_ERR_SHAPE;
  if ((long long)M * K * 2 > kMaxBytes) return WQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(packed) || !aligned16(scales) || !aligned16(zeros))
    return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q2_group(X, packed, scales, zeros, Y, M, K, N, G, as_stream(stream)));
}

int wq_unpack_q2(const void* packed, const int32_t* perm, int8_t* codes, int K, int N, int G,
                 void* stream) {
  if (!packed || !codes) return WQ_ERR_NULL;
  if (int st = check_q2(K, N, G)) return st;
  if (!aligned16(packed)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_q2_unpack(packed, perm, codes, K, N, G, as_stream(stream)));
}

// ------------------------------------------------------------------- W8A8 --

namespace {

// Xq [M, K] and Wq [N, K] are read through 32-bit buffer offsets.
int check_w8a8(int M, int K, int N) {
  if (M < 1 || K < 64 || N < 16 || K % 64 || N % 16) return WQ_ERR_SHAPE;
  if ((long long)K * 127 * 127 >= (1LL << 31)) return WQ_ERR_SHAPE;
  if ((long long)M * K > kMaxBytes || (long long)N * K > kMaxBytes) return WQ_ERR_SHAPE;
  return WQ_OK;
}

int check_ws(int M, int K, int N, const void* ws, size_t ws_bytes) {
  const size_t need = wq::w8a8_workspace_bytes(M, K, N);
  if (need == 0) return WQ_OK;
  if (!ws || ws_bytes < need) return WQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return WQ_ERR_ALIGN;
  return WQ_OK;
}

}  // namespace

size_t wq_workspace_bytes(int op, int M, int K, int N) {
  if (op == WQ_OP_Q8G) {
    if (M < 1 || check_q8(K, N)) return 0;
    return wq::q8_group_workspace_bytes(M, K, N);
  }
  if (op == WQ_OP_Q4G) {
    if (M < 1 || K < 32 || K % 32 || K > 32768 || N < 4 || N % 4) return 0;
    return wq::q4_tiled_workspace_bytes(M, K);
  }
  if (op != WQ_OP_W8A8) return 0;
  if (check_w8a8(M, K, N)) return 0;
  return wq::w8a8_workspace_bytes(M, K, N);
}

int wq_gemm_w8a8(const float* X, const int8_t* Wq, const float* Sw, void* Y, int8_t* Xq,
                 float* Sx, int32_t* acc_out, void* workspace, size_t workspace_bytes, int M, int K,
                 int N, void* stream) {
  if (!X || !Wq || !Sw || !Y || !Xq || !Sx) return WQ_ERR_NULL;
  if (int st = check_w8a8(M, K, N)) return st;
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(Xq) || !aligned16(Sw) || !aligned16(Y) ||
      !aligned16(acc_out))
    return WQ_ERR_ALIGN;
  if (int st = check_ws(M, K, N, workspace, workspace_bytes)) return st;
  return hip_status(wq::launch_w8a8(X, nullptr, Wq, Sw, Y, Xq, Sx, acc_out, workspace, M, K, N,
                                    as_stream(stream)));
}

int wq_gemm_w8a8_noalloc(const float* X, const int8_t* Wq, const float* Sw, void* Y, int8_t* Xq,
                         float* Sx, int32_t* acc_out, int M, int K, int N, void* stream) {
  if (!X || !Wq || !Sw || !Y || !Xq || !Sx) return WQ_ERR_NULL;
  if (int st = check_w8a8(M, K, N)) return st;
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(Xq) || !aligned16(Sw) || !aligned16(Y) ||
      !aligned16(acc_out))
    return WQ_ERR_ALIGN;
  const size_t need = wq::w8a8_workspace_bytes(M, K, N);
  if (need > wq::w8a8_scratch_bytes()) return WQ_ERR_WORKSPACE;
  void* ws = nullptr;
  if (int st = hip_status(wq::w8a8_scratch_ptr(&ws))) return st;
  return hip_status(wq::launch_w8a8(X, nullptr, Wq, Sw, Y, Xq, Sx, acc_out, ws, M, K, N,
                                    as_stream(stream)));
}

int wq_gemm_w8a8_smooth(const float* X, const float* smooth, const int8_t* Wq, const float* Sw,
                        void* Y, int8_t* Xq, float* Sx, int32_t* acc_out, void* workspace,
                        size_t workspace_bytes, int M, int K, int N, void* stream) {
  if (!smooth) return WQ_ERR_NULL;
  if (!aligned16(smooth)) return WQ_ERR_ALIGN;
  if (!X || !Wq || !Sw || !Y || !Xq || !Sx) return WQ_ERR_NULL;
  if (int st = check_w8a8(M, K, N)) return st;
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(Xq) || !aligned16(Sw) || !aligned16(Y) ||
      !aligned16(acc_out))
    return WQ_ERR_ALIGN;
  if (int st = check_ws(M, K, N, workspace, workspace_bytes)) return st;
  return hip_status(wq::launch_w8a8(X, smooth, Wq, Sw, Y, Xq, Sx, acc_out, workspace, M, K, N,
                                    as_stream(stream)));
}

int wq_gemm_int8_mixed(const void* X, const void* W, float threshold, void* Y, int8_t* Xq,
                       float* Sx, int8_t* Wq, float* Sw, float* colmax, uint32_t* outlier_mask,
                       int32_t* outlier_cols, int32_t* n_outlier, int32_t* acc_out,
                       void* workspace, size_t workspace_bytes, int M, int K, int N,
                       void* stream) {
  if (!X || !W || !Y || !Xq || !Sx || !Wq || !Sw || !colmax || !outlier_mask || !outlier_cols ||
      !n_outlier)
    return WQ_ERR_NULL;
  if (int st = check_w8a8(M, K, N)) return st;
  if (threshold != threshold) return WQ_ERR_SHAPE;  // NaN
  if (!aligned16(X) || !aligned16(W) || !aligned16(Xq) || !aligned16(Wq) || !aligned16(Sw) ||
      !aligned16(Y) || !aligned16(colmax) || !aligned16(outlier_mask) || !aligned16(acc_out))
    return WQ_ERR_ALIGN;
  if (int st = check_ws(M, K, N, workspace, workspace_bytes)) return st;
  return hip_status(wq::launch_int8_mixed(X, W, threshold, Y, Xq, Sx, Wq, Sw, colmax,
                                          outlier_mask, outlier_cols, n_outlier, acc_out,
                                          workspace, M, K, N, as_stream(stream)));
}

// ------------------------------------------------------ measurement only --

int wq_calib_empty(int grid, int threads, uint32_t* sink, void* stream) {
  if (!sink) return WQ_ERR_NULL;
  if (grid < 1 || threads < 1 || threads > 1024) return WQ_ERR_SHAPE;
  return hip_status(wq::launch_calib_empty(grid, threads, sink, as_stream(stream)));
}

int wq_calib_stream_read(const void* buf, long long bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return WQ_ERR_NULL;
  if (bytes < 16 || bytes % 16 || bytes > kMaxBytes) return WQ_ERR_SHAPE;
  if (!aligned16(buf)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_calib_stream(buf, (int)bytes, sink, as_stream(stream)));
}

// ------------------------------------------------------------------- misc --

const char* wq_status_str(int status) {
  switch (status) {
    case WQ_OK: return "ok";
    case WQ_ERR_NULL: return "a required pointer is NULL";
    case WQ_ERR_SHAPE: return "invalid shape (size or divisibility rule violated)";
    case WQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case WQ_ERR_DTYPE: return "unknown dtype";
    case WQ_ERR_WORKSPACE: return "workspace missing or smaller than wq_workspace_bytes()";
    case WQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int wq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
