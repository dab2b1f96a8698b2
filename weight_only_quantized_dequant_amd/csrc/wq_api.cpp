// C ABI of libwq.so: argument checks (all before any HIP call), split plans,
// workspace sizing and launches.  Declarations and contracts: include/wq.h.
#include "../../include/wq.h"

#include <hip/hip_runtime.h>

#include <cstdlib>
#include <vector>

#include "wq_internal.h"

namespace wq {

int env_unit_override() {
  const char* v = std::getenv("WQ_SPLITK_UNIT");
  return v ? std::atoi(v) : 0;
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

// Byte extent a buffer-addressed array may have (offsets are 32-bit signed).
constexpr long long kMaxBufferBytes = 0x7FFFFFF0LL;

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_q8(int M, int K, int N, int G) {
  if (M < 1 || K < 32 || N < 16 || G < 32) return WQ_ERR_SHAPE;
  if (K % 32 || G % 32 || K % G || N % 16) return WQ_ERR_SHAPE;
  if ((long long)K * N > kMaxBufferBytes) return WQ_ERR_SHAPE;
  return WQ_OK;
}

int check_q3(int K, int N) {
  if (K < 32 || N < 4 || K % 32 || N % 4) return WQ_ERR_SHAPE;
  if ((long long)(K / 32) * 3 * N * 4 > kMaxBufferBytes) return WQ_ERR_SHAPE;
  return WQ_OK;
}

int check_q4(int M, int K, int N, int G) {
  if (M < 1 || K < 32 || N < 4 || G < 32) return WQ_ERR_SHAPE;
  if (G % 32 || K % G || N % 4) return WQ_ERR_SHAPE;
  if ((long long)(K / 8) * N * 4 > kMaxBufferBytes) return WQ_ERR_SHAPE;
  return WQ_OK;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return WQ_OK;
  if (!ws || have < need) return WQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return WQ_ERR_ALIGN;
  return WQ_OK;
}

}  // namespace

extern "C" {

size_t wq_workspace_bytes(int op, int M, int K, int N, int G) {
  switch (op) {
    case WQ_OP_Q3:
      if (check_q3(K, N) != WQ_OK) return 0;
      return wq::ws_bytes(wq::plan_q3(K, N), N);
    case WQ_OP_Q4G:
      if (check_q4(M, K, N, G) != WQ_OK) return 0;
      return wq::ws_bytes(wq::plan_q4(M, K, N, G), N);
    case WQ_OP_Q8G:
      if (check_q8(M, K, N, G) != WQ_OK) return 0;
      return wq::ws_bytes(wq::plan_q8(M, K, N, G), N);
    default:
      return 0;
  }
}

int wq_matvec_q3(const void* x, const int32_t* qweight, const void* scales, const void* zeros,
                 void* y, int K, int N, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (!x || !qweight || !scales || !zeros || !y) return WQ_ERR_NULL;
  if (dtype != WQ_F32 && dtype != WQ_F16) return WQ_ERR_DTYPE;
  if (int st = check_q3(K, N)) return st;
  if (!aligned16(x) || !aligned16(qweight) || !aligned16(scales)) return WQ_ERR_ALIGN;
  const wq::SplitPlan p = wq::plan_q3(K, N);
  if (int st = check_workspace(workspace, workspace_bytes, wq::ws_bytes(p, N))) return st;
  return hip_status(wq::launch_q3(x, qweight, scales, zeros, y, K, N, dtype == WQ_F16, p,
                                  workspace, as_stream(stream)));
}

int wq_gemm_q8_group(const void* X, const int8_t* qweight, const float* scales, void* Y, int M,
                     int K, int N, int G, void* workspace, size_t workspace_bytes, void* stream) {
  if (!X || !qweight || !scales || !Y) return WQ_ERR_NULL;
  if (int st = check_q8(M, K, N, G)) return st;
  if (!aligned16(X) || !aligned16(qweight) || !aligned16(scales)) return WQ_ERR_ALIGN;
  const wq::SplitPlan p = wq::plan_q8(M, K, N, G);
  if (int st = check_workspace(workspace, workspace_bytes, wq::ws_bytes(p, N))) return st;
  return hip_status(
      wq::launch_q8_group(X, qweight, scales, Y, M, K, N, G, p, workspace, as_stream(stream)));
}

int wq_q4_act_order_perm(const int32_t* g_idx, int K, int G, int32_t* perm) {
  if (!perm) return WQ_ERR_NULL;
  if (K < 1 || G < 1 || K % G) return WQ_ERR_SHAPE;
  const int ng = K / G;
  if (!g_idx) {
    for (int k = 0; k < K; ++k) perm[k] = k;
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
  for (int k = 0; k < K; ++k) perm[next[g_idx[k]]++] = k;  // stable within a group
  return WQ_OK;
}

int wq_q4_prepack(const int32_t* qweight, const int32_t* perm, int32_t* qweight_out, int K, int N,
                  void* stream) {
  if (!qweight || !perm || !qweight_out) return WQ_ERR_NULL;
  if (K < 8 || N < 1 || K % 8) return WQ_ERR_SHAPE;
  const char* a = reinterpret_cast<const char*>(qweight);
  const char* b = reinterpret_cast<const char*>(qweight_out);
  const size_t bytes = (size_t)(K / 8) * N * 4;
  if (a < b + bytes && b < a + bytes) return WQ_ERR_SHAPE;  // overlapping buffers
  return hip_status(wq::launch_q4_prepack(qweight, perm, qweight_out, K, N, as_stream(stream)));
}

int wq_gemm_q4_group(const void* X, const int32_t* qweight, const void* scales,
                     const int32_t* perm, void* Y, int M, int K, int N, int G, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!X || !qweight || !scales || !Y) return WQ_ERR_NULL;
  if (int st = check_q4(M, K, N, G)) return st;
  if (!aligned16(X) || !aligned16(qweight) || !aligned16(scales)) return WQ_ERR_ALIGN;
  const wq::SplitPlan p = wq::plan_q4(M, K, N, G);
  if (int st = check_workspace(workspace, workspace_bytes, wq::ws_bytes(p, N))) return st;
  return hip_status(wq::launch_q4_group(X, qweight, scales, perm, Y, M, K, N, G, p, workspace,
                                        as_stream(stream)));
}

int wq_gemm_w8a8(const float* X, const int8_t* Wq, const float* Sw, void* Y, int8_t* Xq,
                 float* Sx, int32_t* acc_out, int M, int K, int N, void* stream) {
  if (!X || !Wq || !Sw || !Y || !Xq || !Sx) return WQ_ERR_NULL;
  if (M < 1 || K < 64 || N < 16 || K % 64 || N % 16) return WQ_ERR_SHAPE;
  if ((long long)K * 127 * 127 >= (1LL << 31)) return WQ_ERR_SHAPE;
  if ((long long)M * K > kMaxBufferBytes || (long long)N * K > kMaxBufferBytes)
    return WQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(Wq) || !aligned16(Xq)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_w8a8(X, Wq, Sw, Y, Xq, Sx, acc_out, M, K, N, as_stream(stream)));
}

int wq_unpack_q3(const int32_t* qweight, int8_t* codes, int K, int N, void* stream) {
  if (!qweight || !codes) return WQ_ERR_NULL;
  if (int st = check_q3(K, N)) return st;
  if (!aligned16(qweight) || (reinterpret_cast<uintptr_t>(codes) & 3u)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_unpack_q3(qweight, codes, K, N, as_stream(stream)));
}

int wq_unpack_q4(const int32_t* qweight, const int32_t* perm, int8_t* codes, int K, int N,
                 void* stream) {
  if (!qweight || !codes) return WQ_ERR_NULL;
  if (K < 8 || N < 4 || K % 8 || N % 4) return WQ_ERR_SHAPE;
  if (!aligned16(qweight) || (reinterpret_cast<uintptr_t>(codes) & 3u)) return WQ_ERR_ALIGN;
  return hip_status(wq::launch_unpack_q4(qweight, perm, codes, K, N, as_stream(stream)));
}

const char* wq_status_str(int status) {
  switch (status) {
    case WQ_OK: return "ok";
    case WQ_ERR_NULL: return "a required pointer is NULL";
    case WQ_ERR_SHAPE: return "invalid shape (size or divisibility rule violated)";
    case WQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case WQ_ERR_DTYPE: return "unknown dtype";
    case WQ_ERR_WORKSPACE: return "workspace missing or too small";
    case WQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int wq_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
