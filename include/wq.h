/*
 * wq.h - C ABI of the fused dequantize-and-multiply library (libwq.so).
 *
 * The library computes Y = X . dequant(Wq, scales, zeros) for low-bit
 * quantised weights on one AMD MI355X (gfx950) GPU, with the weight codes
 * unpacked and dequantised in registers, never written out as a floating
 * point weight:
 *
 *   - 3-bit GPTQ-style matvec, one scale and one zero per output column
 *     ("GPTQ CUDA kernel walkthrough", yelogs.com, section
 *     "CUDA核函數設計與實現": w = scale * q - zero, codes shifted and masked
 *     out of int32 words, product against a vector);
 *   - 4-bit symmetric group-wise GEMM with an act-order row -> group map
 *     ("GPTQ算法解析", intelliparadigm.com, section 4.1: w_bit 4, group 128,
 *     sym, act_order; "Quantization CUDA", tom-jerr.github.io, sections
 *     "量化粒度" and "Int4 Weight Only Quantization");
 *   - int8 symmetric group-wise weight-only GEMV / small-batch GEMM
 *     ("Quantization CUDA", section "Int8 Weight Only Quantization":
 *     Y = X.(Wint*Sw) = (X.Wint)*Sw with fp32 accumulation;
 *     "融合反量化与GEMM：LLM推理的CUDA内核优化实践", zingnex.cn, section
 *     "技术实现细节": one fp32 scale per 128 rows of K per column);
 *   - W8A8 dynamic-quantisation GEMM ("Quantization CUDA", sections
 *     "Dynamic Quantization" and "优化": activations quantised at run time,
 *     int8 multiply, int32 accumulation, Y = Sx * (Xint.Wint) * Sw with the
 *     rescale fused after the accumulation and a bf16 result).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Memory: every array argument is a DEVICE pointer owned by the caller,
 *   except where an argument is marked HOST.  The library never allocates or
 *   frees memory, never synchronises a stream, and never changes the current
 *   device; work runs on the device that owns the buffers, on `stream`
 *   (a hipStream_t; NULL means the default stream), asynchronously.
 * - Layout: row-major and contiguous.  Packed weights keep N (the output
 *   column) contiguous; codes are packed along K.
 * - Outputs are overwritten, never accumulated into.
 * - Alignment: packed weights, X/x and scales must be 16-byte aligned.
 * - Errors: every call returns a wq_status_t.  Argument checks run on the
 *   host before any HIP call; a failed check launches nothing.  A launch
 *   failure returns WQ_ERR_HIP (the hipError_t is kept per thread, see
 *   wq_last_hip_error).  A fault inside a kernel surfaces at the caller's next
 *   synchronisation, as for any HIP library.  Nothing throws or aborts.
 * - Workspace: the weight-only products split K across workgroups and need a
 *   device workspace of wq_workspace_bytes(...) bytes for the partial sums and
 *   the per-tile arrival counters.  It must be zero-filled once after
 *   allocation; every call leaves it zero-filled again.  Calls that may run
 *   concurrently (different streams) need distinct workspaces.
 * - Results are bitwise reproducible for a given shape: every reduction runs
 *   in a fixed order.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wq_status {
  WQ_OK = 0,
  WQ_ERR_NULL = 1,      /* a required pointer is NULL                         */
  WQ_ERR_SHAPE = 2,     /* a size or divisibility rule is violated            */
  WQ_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned                   */
  WQ_ERR_DTYPE = 4,     /* unknown dtype code                                 */
  WQ_ERR_WORKSPACE = 5, /* workspace missing or smaller than required         */
  WQ_ERR_HIP = 6        /* a HIP runtime call failed; see wq_last_hip_error() */
} wq_status_t;

typedef enum wq_dtype {
  WQ_F32 = 0,
  WQ_F16 = 1
} wq_dtype_t;

typedef enum wq_op {
  WQ_OP_Q3 = 0,   /* wq_matvec_q3      */
  WQ_OP_Q4G = 1,  /* wq_gemm_q4_group  */
  WQ_OP_Q8G = 2   /* wq_gemm_q8_group  */
} wq_op_t;

/* Workspace bytes needed by `op` at this shape (M rows of X, K, N, group
 * size G; M and G are ignored where they do not apply).  Returns 0 for an
 * invalid op or shape.  The size is a pure function of its arguments. */
size_t wq_workspace_bytes(int op, int M, int K, int N, int G);

/* 3-bit matvec:  y[n] = sum_k x[k] * (scale[n] * q[k, n] - zero[n]).
 *
 * x       [K]           dtype (fp32 or fp16)
 * qweight [3K/32, N]    int32; for column n and 32-row block b, the words
 *                       3b, 3b+1, 3b+2 form a 96-bit little-endian value whose
 *                       bits 3i..3i+2 hold the code q (0..7) of row 32b + i.
 * scales  [N], zeros [N]  dtype; zero is the stored per-column offset
 *                       (w = scale*q - zero, the form of the page above).
 * y       [N]           dtype, written.
 * dtype   WQ_F32 or WQ_F16 (x, scales, zeros and y share it).  Accumulation
 *         is fp32 in both cases.
 * Rules:  K % 32 == 0, K >= 32, N % 4 == 0, N >= 4.
 */
int wq_matvec_q3(const void* x, const int32_t* qweight, const void* scales,
                 const void* zeros, void* y, int K, int N, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Group-wise int8 weight-only GEMM / GEMV:
 *   Y[m, n] = sum_k X[m, k] * (scale[k / G, n] * q[k, n]).
 *
 * X       [M, K]  fp16;   qweight [K, N] int8 (codes -127..127 symmetric);
 * scales  [K/G, N] fp32;  Y [M, N] fp16, written (fp32 accumulation, one
 *         round-to-nearest-even to fp16 at the end).
 * Rules:  M >= 1, K % 32 == 0, G % 32 == 0, K % G == 0, N % 16 == 0.
 */
int wq_gemm_q8_group(const void* X, const int8_t* qweight, const float* scales,
                     void* Y, int M, int K, int N, int G,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Act-order preparation, step 1 (HOST arrays, runs on the CPU):
 * from g_idx[K] (row k belongs to group g_idx[k]) build perm[K], the K rows
 * listed group by group (rows of group 0 in increasing k, then group 1, ...).
 * g_idx == NULL means g_idx[k] = k / G (then perm is the identity).
 * Returns WQ_ERR_SHAPE unless every group 0..K/G-1 owns exactly G rows (the
 * shape act-order quantisation produces). */
int wq_q4_act_order_perm(const int32_t* g_idx, int K, int G, int32_t* perm);

/* Act-order preparation, step 2 (device): reorder the rows of a 4-bit weight
 * into the order perm lists.  qweight_out row i (nibble i % 8 of word i / 8)
 * receives the code of original row perm[i].  qweight and qweight_out are
 * [K/8, N] int32 in the 4-bit layout of wq_gemm_q4_group and must not
 * overlap.  Rules: K % 8 == 0, N >= 1. */
int wq_q4_prepack(const int32_t* qweight, const int32_t* perm, int32_t* qweight_out,
                  int K, int N, void* stream);

/* Group-wise 4-bit GEMM (symmetric, optional act-order):
 *   Y[m, n] = sum_i X[m, perm[i]] * scale[i / G, n] * q'[i, n]
 * where q' is the prepacked weight (rows in perm order, so rows
 * [gG, gG + G) all belong to group g).  With perm == NULL the weight is used
 * as stored and row k belongs to group k / G.
 *
 * X       [M, K]   fp16;
 * qweight [K/8, N] int32, row 8r + j in nibble j (bits 4j..4j+3) of word r,
 *                  stored as u = q + 8 (q in -8..7);
 * scales  [K/G, N] fp16;  perm [K] int32 device array or NULL;
 * Y       [M, N]   fp16, written (fp32 accumulation).
 * Rules:  M >= 1, K % G == 0, G % 32 == 0, N % 4 == 0.
 */
int wq_gemm_q4_group(const void* X, const int32_t* qweight, const void* scales,
                     const int32_t* perm, void* Y, int M, int K, int N, int G,
                     void* workspace, size_t workspace_bytes, void* stream);

/* W8A8 dynamic-quantisation GEMM:
 *   a[m] = max_k |X[m, k]|;  Sx[m] = a[m] / 127 (fp32, round to nearest);
 *   Xq[m, k] = clamp(rint(X[m, k] / Sx[m]), -127, 127)  (0 when a[m] == 0);
 *   acc[m, n] = sum_k Xq[m, k] * Wq[n, k]   (exact int32);
 *   Y[m, n] = bf16_rne( (Sx[m] * float(acc)) * Sw[n] )  (two fp32 multiplies).
 *
 * X   [M, K] fp32;  Wq [N, K] int8 (quantised offline, K contiguous);
 * Sw  [N] fp32 per-output-channel scale;  Y [M, N] bf16 (uint16 bits), written;
 * Xq  [M, K] int8 and Sx [M] fp32: written (the run-time quantised X);
 * acc_out [M, N] int32: written when non-NULL (for checking), else the
 *         accumulator never leaves the chip.
 * Two launches on `stream` (quantiser, then GEMM).
 * Rules:  M >= 1, K % 64 == 0, N % 16 == 0, and K * 127 * 127 < 2^31.
 */
int wq_gemm_w8a8(const float* X, const int8_t* Wq, const float* Sw, void* Y,
                 int8_t* Xq, float* Sx, int32_t* acc_out, int M, int K, int N,
                 void* stream);

/* Bit-exact unpack checks: write the signed codes as int8 [K, N], through the
 * same device extraction routines the fused kernels use.
 * wq_unpack_q3: codes 0..7 from the 3-bit layout.  Rules: K % 32 == 0, N % 4 == 0.
 * wq_unpack_q4: codes q = u - 8 of the 4-bit layout; when perm is non-NULL the
 *   input is a prepacked weight and row i is written to codes row perm[i]
 *   (undoing the reorder).  Rules: K % 8 == 0, N % 4 == 0. */
int wq_unpack_q3(const int32_t* qweight, int8_t* codes, int K, int N, void* stream);
int wq_unpack_q4(const int32_t* qweight, const int32_t* perm, int8_t* codes,
                 int K, int N, void* stream);

/* Static text for a status code. */
const char* wq_status_str(int status);

/* The hipError_t behind this thread's most recent WQ_ERR_HIP (0 if none). */
int wq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
