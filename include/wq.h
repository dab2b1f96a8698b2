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
 * Weight layouts
 * --------------
 * The weight-only products read a copy of the weight that wq_prepack_*
 * writes once, offline (the weights are constant; "Quantization CUDA",
 * section "Marlin 格式", re-lays quantised weights out the same way for its
 * kernel).  The copy holds exactly the same codes, regrouped into column
 * panels over the whole of K in the order the GPU threads read them, so one
 * workgroup computes a panel of outputs alone and every load of a wave is
 * contiguous.  Its size is wq_packed_bytes(); it is opaque, and only valid
 * for the (op, K, N, G) it was made for.  wq_unpack_* read it back to plain
 * codes through the same register-level extraction the products use.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Memory: every array argument is a DEVICE pointer owned by the caller,
 *   except where an argument is marked HOST.  The library never allocates or
 *   frees memory, never synchronises a stream, and never changes the current
 *   device; work runs on the device that owns the buffers, on `stream`
 *   (a hipStream_t; NULL means the default stream), asynchronously.  The
 *   int8 and 4-bit products above 32 and 4 rows of X and the W8A8 family take a workspace,
 *   sized by wq_workspace_bytes(), in which a call leaves nothing that a
 *   later call depends on (it needs no clearing); the other products need
 *   none (no partial result leaves a workgroup).  Calls that overlap in time
 *   need separate workspaces.
 * - Layout: row-major and contiguous.  Stored (unpacked) weights keep N (the
 *   output column) contiguous; codes are packed along K.
 * - Outputs are overwritten, never accumulated into.
 * - Alignment: weights (plain and packed), X/x and scales must be 16-byte
 *   aligned; so must g_idx-derived permutation arrays.
 * - Errors: every call returns a wq_status_t.  Argument checks run on the
 *   host before any HIP call; a failed check launches nothing.  A launch
 *   failure returns WQ_ERR_HIP (the hipError_t is kept per thread, see
 *   wq_last_hip_error).  A fault inside a kernel surfaces at the caller's next
 *   synchronisation, as for any HIP library.  Nothing throws or aborts.
 * - Results are bitwise reproducible for a given shape: every reduction runs
 *   in a fixed order.  Calls are re-entrant and may run concurrently.
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
  WQ_ERR_WORKSPACE = 5, /* workspace NULL or smaller than wq_workspace_bytes() */
  WQ_ERR_HIP = 6        /* a HIP runtime call failed; see wq_last_hip_error() */
} wq_status_t;

typedef enum wq_dtype {
  WQ_F32 = 0,
  WQ_F16 = 1
} wq_dtype_t;

typedef enum wq_op {
  WQ_OP_Q3 = 0,   /* 3-bit matvec              */
  WQ_OP_Q4G = 1,  /* 4-bit group-wise GEMM      */
  WQ_OP_Q8G = 2,  /* int8 group-wise GEMV/GEMM  */
  WQ_OP_Q2G = 3,  /* 2-bit group-wise GEMM      */
  WQ_OP_W8A8 = 4  /* W8A8 GEMM (also SmoothQuant and LLM.int8()) */
} wq_op_t;

/* Bytes of the packed weight for `op` at this shape (G is used by
 * WQ_OP_Q4G and WQ_OP_Q2G only).  Returns 0 for an invalid op or shape.  Pure function. */
size_t wq_packed_bytes(int op, int K, int N, int G);

/* Bytes of device workspace a call of `op` needs at this shape; 0 when it
 * needs none.
 * - WQ_OP_W8A8 (wq_gemm_w8a8, wq_gemm_w8a8_smooth, wq_gemm_int8_mixed): when
 *   the GEMM splits K over workgroups it keeps S int32 partial tiles,
 *   S * M * N * 4 bytes (S = 2 at M = 256, K = N = 8192: 16 MiB; S = 1, no
 *   workspace, once the 128 x 128 output tiles alone fill the GPU, e.g. for
 *   M > 256 at N = 8192).
 * - WQ_OP_Q8G (wq_gemm_q8_group): above 32 rows of X, while the 32 x 128
 *   output tiles alone do not fill the GPU, the fp32 partial tiles of S K
 *   slices, S * M * N * 4 bytes (S = 8 for 33 <= M <= 64 at K = N = 4096;
 *   the size holds for every group size the tiled path takes).
 * - WQ_OP_Q4G (wq_gemm_q4_group, wq_gemm_q4_group_zp): above 4 rows of X,
 *   X in the packed weight's row order, Mp * Kp * 2 bytes (Mp = M rounded
 *   up to 16, Kp = K rounded up to 128).
 * - The other ops never need one (no partial result leaves a workgroup).
 * Returns 0 for an invalid shape.  Pure function. */
size_t wq_workspace_bytes(int op, int M, int K, int N);

/* ---------------------------------------------------------------- 3-bit -- */

/* Re-lay out a 3-bit weight.
 * qweight [3K/32, N] int32: for column n and 32-row block b, the words
 *   3b, 3b+1, 3b+2 form a 96-bit little-endian value whose bits 3i..3i+2 hold
 *   the code q (0..7) of row 32b + i.
 * packed: wq_packed_bytes(WQ_OP_Q3, K, N, 0) bytes, written.
 * Rules: K % 32 == 0, K >= 32, N % 4 == 0, N >= 4. */
int wq_prepack_q3(const int32_t* qweight, void* packed, int K, int N, void* stream);

/* 3-bit matvec ("GPTQ CUDA kernel walkthrough", yelogs.com, section
 * "CUDA核函數設計與實現": 32 three-bit codes per 3 int32 words, each code
 * shifted and masked out, dequantised as scale * q - zero with one scale and
 * one zero per output column, and multiplied into the vector; the fp16 form
 * is that page's half2 path):
 *   y[n] = sum_k x[k] * (scale[n] * q[k, n] - zero[n]).
 * x [K], scales [N], zeros [N], y [N] (written) share `dtype` (WQ_F32 or
 * WQ_F16); zero is the stored per-column offset (w = scale*q - zero).
 * Accumulation is fp32 in both cases; the fp16 result is rounded once, to
 * nearest even.  Any finite x is taken as given (no step scales it up, so
 * y is finite whenever the fp32 sums are).  packed: from wq_prepack_q3 at
 * the same (K, N).
 * Rules: as wq_prepack_q3, and K <= 32768 (fp16) / 16384 (fp32). */
int wq_matvec_q3(const void* x, const void* packed, const void* scales, const void* zeros,
                 void* y, int K, int N, int dtype, void* stream);

/* ----------------------------------------------------------------- int8 -- */

/* Re-lay out a group-wise int8 weight qweight [K, N] (codes -127..127) into
 * column pairs of 16-byte pieces (8 rows x 2 columns, K/8 pieces per pair).
 * packed: wq_packed_bytes(WQ_OP_Q8G, K, N, G) = K * N bytes, written.
 * Rules: K % 32 == 0, N % 16 == 0. */
int wq_prepack_q8(const int8_t* qweight, void* packed, int K, int N, void* stream);

/* Group-wise int8 weight-only GEMM / GEMV:
 *   Y[m, n] = sum_k X[m, k] * (scale[k / G, n] * q[k, n]).
 * X [M, K] fp16; packed: from wq_prepack_q8; scales [K/G, N] fp32;
 * Y [M, N] fp16, written (fp32 accumulation, one round to nearest even).
 * Evaluated per group as scale * (sum of X * q), exact products, fp32 sums.
 * M <= 32, or G not a multiple of 64: streaming passes over the packed
 * weight, one per 32 rows of X (one or two rows on v_dot2, 3 to 32 on the
 * matrix cores).  Otherwise a tiled matrix-core
 * launch (32 x 128 output tiles) reads the packed weight once; while those
 * tiles alone do not fill the GPU (e.g. M <= 64 at N = 4096) K is split over
 * 2..8 workgroups per tile, their fp32 partial tiles go to the workspace, and
 * a second launch adds them in a fixed order and rounds once.
 * ("Quantization CUDA", tom-jerr.github.io, "Int8 Weight Only Quantization";
 * "融合反量化与GEMM：LLM推理的CUDA内核优化实践", zingnex.cn, "技术实现细节".)
 * workspace: device, needed when G % 64 == 0 and wq_workspace_bytes(
 *   WQ_OP_Q8G, M, K, N) > 0 (S * M * N * 4 bytes, S the number of K slices:
 *   8 for 33 <= M <= 64 at K = N = 4096), else NULL allowed; 16-byte aligned;
 *   needs no clearing.  WQ_ERR_WORKSPACE if missing or too small.  Calls
 *   that overlap in time need separate workspaces.
 * Rules: M >= 1, K % 32 == 0, N % 16 == 0, G % 32 == 0, K % G == 0,
 * M * K * 2 < 2^31; Y 16-byte aligned as well. */
int wq_gemm_q8_group(const void* X, const void* packed, const float* scales, void* Y, int M,
                     int K, int N, int G, void* workspace, size_t workspace_bytes, void* stream);

/* The separated (unfused) form's first step, for comparison with the fused
 * product ("融合反量化与GEMM：LLM推理的CUDA内核优化实践", zingnex.cn, section
 * "CUDA内核架构": a standalone INT8 -> FP32 dequantisation kernel that
 * writes the whole weight, followed by a general GEMM; section "性能对比数据",
 * the "CUDA分离" row): materialise
 *   W[k, n] = scale[k / G, n] * q[k, n]
 * as one fp32 multiply per weight; with dtype WQ_F16 that fp32 product is
 * rounded once more, to nearest even.  qweight [K, N] int8 (the stored
 * codes, not the packed copy), scales [K/G, N] fp32, W [K, N] fp32 or fp16,
 * written.  A GEMM of the caller's choice then multiplies X by W.
 * Rules: K % 32 == 0, N % 16 == 0, G % 32 == 0, K % G == 0,
 * K * N * sizeof(W) < 2^31; all arrays 16-byte aligned. */
int wq_dequant_q8_group(const int8_t* qweight, const float* scales, void* W, int K, int N, int G,
                        int dtype, void* stream);

/* ---------------------------------------------------------------- 4-bit -- */

/* Act-order preparation (HOST arrays, runs on the CPU): from g_idx[K] (row k
 * belongs to group g_idx[k]) build perm[K], the rows listed group by group
 * (rows of group 0 in increasing k, then group 1, ...), and its inverse
 * invperm[K] (invperm[perm[i]] = i).  g_idx == NULL means g_idx[k] = k / G.
 * Returns WQ_ERR_SHAPE unless every group 0..K/G-1 owns exactly G rows (the
 * shape act-order quantisation produces). */
int wq_q4_act_order_perm(const int32_t* g_idx, int K, int G, int32_t* perm, int32_t* invperm);

/* Re-lay out a 4-bit weight qweight [K/8, N] int32 (row 8r + j in nibble j,
 * bits 4j..4j+3, of word r, stored as u = q + 8), its rows taken in the
 * order perm lists (device array [K], or NULL for the stored order).
 * perm must be a permutation of 0..K-1 (wq_q4_act_order_perm builds one);
 * the library does not copy it back to check: entries outside 0..K-1 are
 * skipped, never used as addresses, and a perm that repeats rows leaves
 * the packed weight undefined (but every access in bounds).
 * packed: wq_packed_bytes(WQ_OP_Q4G, K, N, G) bytes, written.
 * The packed weight also holds the inverse of perm as a table of K uint16,
 * and perm itself as a table of K rounded up to 128 uint16 (0xFFFF past K).
 * Rules: K % G == 0, G a power of two >= 32, K <= 32768, N % 4 == 0. */
int wq_prepack_q4(const int32_t* qweight, const int32_t* perm, void* packed, int K, int N, int G,
                  void* stream);

/* Group-wise 4-bit GEMM (symmetric, optional act-order)
 * ("Quantization CUDA", tom-jerr.github.io, sections "Int4 Weight Only
 * Quantization" and "量化粒度": int4 codes packed along K, one scale per group
 * of 128 rows; "GPTQ算法解析", intelliparadigm.com, section 4.1: act_order,
 * a row -> group map g_idx that is not monotone in K):
 *   Y[m, n] = sum_k X[m, k] * scale[g_idx[k], n] * q[k, n]
 * computed from the packed weight (rows in perm order) as
 *   sum_i X[m, perm[i]] * scale[i / G, n] * q[perm[i], n].
 * X [M, K] fp16; packed: from wq_prepack_q4 (the row order perm travels
 * inside it); scales [K/G, N] fp16; Y [M, N] fp16, written (fp32
 * accumulation).
 * Up to 4 rows: one launch, X staged whole in LDS, no
 * workspace.  More rows: X is first gathered into the packed weight's row
 * order in the workspace (in matrix-core operand order), then one launch
 * per 64 rows (48 for groups of 64, 32 for groups of 32) reads the packed
 * weight once (16-row matrix-core tiles).
 * workspace: device, workspace_bytes >= wq_workspace_bytes(WQ_OP_Q4G, M, K,
 *   N) = Mp * Kp * 2 bytes when M > 4 (Mp = M rounded up to 16, Kp = K
 *   rounded up to 128), else 0 (NULL allowed); 16-byte aligned; needs no
 *   clearing.  WQ_ERR_WORKSPACE if missing or too small.  Calls that overlap
 *   in time need separate workspaces.
 * Rules: as wq_prepack_q4, M >= 1, M * K * 2 < 2^31. */
int wq_gemm_q4_group(const void* X, const void* packed, const void* scales, void* Y, int M, int K,
                     int N, int G, void* workspace, size_t workspace_bytes, void* stream);

/* Asymmetric (AWQ-style) group-wise 4-bit GEMM:
 *   Y[m, n] = sum_k X[m, k] * (u[k, n] - zero[g, n]) * scale[g, n],
 *   g = g_idx[k] (through the row order inside the packed weight) or k / G,
 * with u the stored unsigned nibble 0..15 (the same packed weight as
 * wq_gemm_q4_group: wq_prepack_q4 stores the nibbles as given).
 * ("Quantization CUDA", tom-jerr.github.io, section "量化粒度": x = S (q - Z),
 * each group its own S and Z; section "Marlin 格式": the asymmetric step
 * W_fp16 = (W_int4 - Zero) * Scale.)
 * X [M, K] fp16; scales and zeros [K/G, N] fp16 (zeros as values, e.g. the
 * integers 0..15); Y [M, N] fp16, written (fp32 accumulation; the zero is
 * applied once per group to the accumulated sums); workspace as
 * wq_gemm_q4_group.
 * Rules: as wq_gemm_q4_group; zeros 16-byte aligned. */
int wq_gemm_q4_group_zp(const void* X, const void* packed, const void* scales, const void* zeros,
                        void* Y, int M, int K, int N, int G, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- 2-bit -- */

/* Re-lay out a 2-bit weight qweight [K/16, N] int32 (row 16r + j in bits
 * 2j, 2j+1 of word r, unsigned values 0..3), its rows taken in the order
 * perm lists (device array [K], from wq_q4_act_order_perm, or NULL for the
 * stored order; a permutation of 0..K-1, as for wq_prepack_q4).  packed: wq_packed_bytes(WQ_OP_Q2G, K, N, G) bytes, written;
 * it also holds the inverse of perm as a table of K uint16.
 * Rules: K % G == 0, G a power of two >= 32, K <= 32768, N % 4 == 0. */
int wq_prepack_q2(const int32_t* qweight, const int32_t* perm, void* packed, int K, int N, int G,
                  void* stream);

/* Asymmetric group-wise 2-bit GEMM:
 *   Y[m, n] = sum_k X[m, k] * (u[k, n] - zero[g, n]) * scale[g, n],
 *   g = g_idx[k] (through the row order inside the packed weight) or k / G,
 * u the stored value 0..3.  ("GPTQ CUDA kernel walkthrough", yelogs.com:
 * 2-bit codes as a lower bit width to support; "Quantization CUDA",
 * tom-jerr.github.io, section "量化粒度": x = S (q - Z), each group its own S
 * and Z.)  X [M, K] fp16; packed: from wq_prepack_q2; scales and zeros
 * [K/G, N] fp16; Y [M, N] fp16, written (fp32 accumulation; the zero is
 * applied once per group to the accumulated sums).
 * Rules: as wq_prepack_q2, M >= 1; X, packed, scales and zeros 16-byte
 * aligned. */
int wq_gemm_q2_group_zp(const void* X, const void* packed, const void* scales, const void* zeros,
                        void* Y, int M, int K, int N, int G, void* stream);

/* ----------------------------------------------------------------- W8A8 -- */

/* W8A8 dynamic-quantisation GEMM ("Quantization CUDA", tom-jerr.github.io,
 * section "Dynamic Quantization": Y = X.W = (Sx*Xint).(Wint*Sw) =
 * Sx*(Xint.Wint)*Sw, activations quantised per token at run time, weights
 * per output channel in preprocessing, int8 products accumulated in int32;
 * section "优化": the rescale fused after the accumulation, bf16 result):
 *   a[m] = max_k |X[m, k]|;  Sx[m] = a[m] / 127 (fp32, round to nearest);
 *   Xq[m, k] = clamp(rint(X[m, k] / Sx[m]), -127, 127)  (0 when a[m] == 0);
 *   acc[m, n] = sum_k Xq[m, k] * Wq[n, k]   (exact int32);
 *   Y[m, n] = bf16_rne( (Sx[m] * float(acc)) * Sw[n] )  (two fp32 multiplies).
 * X [M, K] fp32;  Wq [N, K] int8 (quantised offline, K contiguous);
 * Sw [N] fp32 per-output-channel scale;  Y [M, N] bf16 (uint16 bits), written;
 * Xq [M, K] int8 and Sx [M] fp32: written (the run-time quantised X);
 * acc_out [M, N] int32: written when non-NULL (for checking), else the
 *   accumulator never reaches memory except as the split-K partials.
 * workspace: device, workspace_bytes >= wq_workspace_bytes(WQ_OP_W8A8, M,
 *   K, N) (may be NULL when that is 0), 16-byte aligned; scratch for the
 *   int32 partial tiles of the K slices, summed in a fixed order, so the
 *   result is bit-identical for any workspace.  WQ_ERR_WORKSPACE if missing
 *   or too small.
 * Two or three launches on `stream` (quantiser; GEMM; with a split K, the
 * sum of the partials and the rescale).
 * Rules: M >= 1, K % 64 == 0, N % 16 == 0, K * 127 * 127 < 2^31,
 * M * K < 2^31, N * K < 2^31; X, Wq, Sw, Y, Xq and acc_out (when given)
 * 16-byte aligned. */
int wq_gemm_w8a8(const float* X, const int8_t* Wq, const float* Sw, void* Y, int8_t* Xq,
                 float* Sx, int32_t* acc_out, void* workspace, size_t workspace_bytes, int M,
                 int K, int N, void* stream);

/* wq_gemm_w8a8 for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation and results, with the workspace taken from a device array the
 * library holds on each GPU it runs on (16 MiB per GPU, kept until the
 * process ends; its address is looked up once per device, with that device
 * current).  Allocates and frees nothing.  Arguments and rules as
 * wq_gemm_w8a8 without workspace; WQ_ERR_WORKSPACE when the shape needs
 * more than 16 MiB (wq_workspace_bytes(WQ_OP_W8A8, M, K, N) > 16 MiB; e.g.
 * M = 256, K = N = 8192 needs exactly 16 MiB).  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams,
 * other threads) race and give undefined results; calls ordered on one
 * stream are safe.  Nothing in the array needs clearing: each call writes
 * every partial it reads. */
int wq_gemm_w8a8_noalloc(const float* X, const int8_t* Wq, const float* Sw, void* Y, int8_t* Xq,
                         float* Sx, int32_t* acc_out, int M, int K, int N, void* stream);

/* SmoothQuant around the same W8A8 step:  Y = (X diag(s)^-1) . (diag(s) W).
 * The activation side runs here: the row quantiser works on X[m, k] / s[k]
 * (one IEEE fp32 division per element) and writes Xq and Sx of that matrix;
 * everything else is wq_gemm_w8a8.  The weight side is folded offline: Wq and
 * Sw must quantise diag(s) W (rows of W indexed by k scaled by s[k]).
 * ("Quantization CUDA", tom-jerr.github.io, section "Smoothquant".)
 * smooth [K] fp32, s[k] > 0, 16-byte aligned; other arguments and rules as
 * wq_gemm_w8a8. */
int wq_gemm_w8a8_smooth(const float* X, const float* smooth, const int8_t* Wq, const float* Sw,
                        void* Y, int8_t* Xq, float* Sx, int32_t* acc_out, void* workspace,
                        size_t workspace_bytes, int M, int K, int N, void* stream);

/* LLM.int8() mixed-precision decomposition of Y = X . W^T
 * ("Quantization CUDA", tom-jerr.github.io, section "LLM.int8()": the
 * activations are scanned against a magnitude threshold such as 6.0; the
 * columns of X holding such values and the matching weight entries stay in
 * fp16 and are multiplied in fp16; the rest of X is quantised per token and
 * the rest of W per output channel to int8 and multiplied in int8; the int8
 * result, rescaled, and the fp16 product are added):
 *   colmax[k] = max_m |X[m, k]|;  column k is an outlier when colmax[k] > threshold;
 *   Xq, Sx: each row of X with the outlier columns set to 0, quantised as in
 *     wq_gemm_w8a8 (Sx = absmax / 127, codes clamp(rint(x / Sx), -127, 127));
 *   Wq, Sw: each row n of W (output channel n) with the outlier columns set
 *     to 0, quantised by the same rule (Sw over the regular columns only);
 *   acc = Xq . Wq^T (exact int32);
 *   o[m, n] = sum over outlier columns k of X[m, k] * W[n, k] (fp32; each
 *     product of two fp16 values is exact);
 *   Y[m, n] = fp16_rne( (Sx[m] * float(acc)) * Sw[n] + o[m, n] ).
 * X [M, K] fp16; W [N, K] fp16 (K contiguous, row n = output channel n);
 * Y [M, N] fp16, written.  Written as well: Xq [M, K] int8, Sx [M] fp32,
 * Wq [N, K] int8, Sw [N] fp32 (the quantised regular part), colmax [K] fp32,
 * outlier_mask [K / 32] uint32 (bit k % 32 of word k / 32 set for an outlier
 * column), outlier_cols [K] int32 (the first *n_outlier entries, ascending)
 * and n_outlier [1] int32; acc_out and workspace as wq_gemm_w8a8.  The
 * weight is read in fp16 and quantised on every call because its split
 * depends on X.  Three or four launches on `stream` (column scan; quantiser
 * of the rows of X and W and the outlier list; GEMM; with a split K, the
 * sum of the partials; the fp16 side joins the rescale).
 * Rules: M >= 1, K % 64 == 0, N % 16 == 0, K * 127 * 127 < 2^31, threshold
 * not NaN; X, W, Y, Xq, Wq, Sw, colmax, outlier_mask and acc_out (when
 * given) 16-byte aligned. */
int wq_gemm_int8_mixed(const void* X, const void* W, float threshold, void* Y, int8_t* Xq,
                       float* Sx, int8_t* Wq, float* Sw, float* colmax, uint32_t* outlier_mask,
                       int32_t* outlier_cols, int32_t* n_outlier, int32_t* acc_out,
                       void* workspace, size_t workspace_bytes, int M, int K, int N,
                       void* stream);

/* ------------------------------------------------------ bit-exact checks -- */

/* Write the signed codes a packed weight holds as int8 [K, N], through the
 * same device extraction routines the products use.
 * wq_unpack_q3: codes 0..7.  wq_unpack_q8: codes -127..127.
 * wq_unpack_q4: codes q = u - 8, in the original row order (perm as given to
 *   wq_prepack_q4, or NULL). */
int wq_unpack_q3(const void* packed, int8_t* codes, int K, int N, void* stream);
int wq_unpack_q8(const void* packed, int8_t* codes, int K, int N, void* stream);
int wq_unpack_q4(const void* packed, const int32_t* perm, int8_t* codes, int K, int N, int G,
                 void* stream);
/* wq_unpack_q2: the values u (0..3) in the original row order. */
int wq_unpack_q2(const void* packed, const int32_t* perm, int8_t* codes, int K, int N, int G,
                 void* stream);

/* ---------------------------------------------------- measurement only -- */

/* References for timing the streaming products; neither computes anything
 * and no product calls them.  They sit in the library so that the dispatch
 * floor and the streaming ceiling are measured through the same build, launch
 * path and loads as the products they are compared with.
 * wq_calib_empty: one launch of an empty kernel, grid x threads (1..1024),
 *   that touches no memory: the dispatch floor of a launch.
 * wq_calib_stream_read: one launch that reads bytes [0, bytes) of buf once
 *   with the int8 GEMV's weight-stream loads (512-thread workgroups, eight
 *   16-byte non-temporal buffer loads per thread, 64 KiB per workgroup) and
 *   discards them: the achievable time for any kernel that reads those bytes.
 *   buf: device, 16-byte aligned; bytes % 16 == 0, 16 <= bytes < 2^31.
 *   sink: device uint32 [1]; written only if the xor of all words read
 *   equals 0x9E3779B9 (its value carries no meaning).
 * Errors: WQ_ERR_NULL, WQ_ERR_SHAPE, WQ_ERR_ALIGN, WQ_ERR_HIP as above. */
int wq_calib_empty(int grid, int threads, uint32_t* sink, void* stream);
int wq_calib_stream_read(const void* buf, long long bytes, uint32_t* sink, void* stream);

/* Static text for a status code. */
const char* wq_status_str(int status);

/* The hipError_t behind this thread's most recent WQ_ERR_HIP (0 if none). */
int wq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
