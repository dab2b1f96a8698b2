// Device helpers shared by the fused dequantize-and-multiply kernels (gfx950).
//
// Code -> fp16 conversion without arithmetic.  A 32-bit register whose two
// halves have a zero exponent field and an integer v (< 1024) in the mantissa
// is the pair of fp16 subnormals (v_lo * 2^-24, v_hi * 2^-24), exactly.  So a
// packed code masked into the mantissa of each half (one v_and_b32, or one
// v_perm_b32 for bytes) is already an exact fp16 pair, and v_dot2_f32_f16
// (which keeps fp16 subnormals: checked on gfx950) multiplies it with a pair
// of fp16 activations and accumulates in fp32.  The 2^-24 and any bit offset
// 2^p of the code inside the mantissa are powers of two, folded into one
// scale at the end.  Products of an fp16 activation and a code of at most 8
// bits are exact in fp32, so only the fp32 accumulation rounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kTwo24 = 16777216.0f;      // 2^24: undoes the subnormal scale

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
// Takes its argument by value on purpose: __builtin_bit_cast applied directly
// to an element of an ext_vector_type reads the vector's first element.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }

// Buffer-resource view of a read-only array of `bytes` bytes (< 2^31).  A
// raw buffer load whose offset falls outside the range returns zeros, which
// is how ragged tiles read past the edge of a weight without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// 128-bit non-temporal buffer load (cache policy "nt": data used once).
__device__ __forceinline__ u32x4 buffer_stream(__amdgpu_buffer_rsrc_t r, int offset) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 2);
}
// Offset that is always out of range: the load returns zeros.
constexpr int kOutOfRange = 0x7FFFFFF0;

// Part r of a contiguous split of n items into g parts, with q = n / g and
// e = n % g worked out on the host: part r takes q + 1 items if r < e, else
// q, and the parts follow each other in order.  (Two scalar multiplies; the
// division n * r / g in the kernel costs a 64-bit software divide before the
// first load can be addressed.)
struct SplitPart {
  int begin, count;
};
__device__ __forceinline__ SplitPart split_part(int r, int q, int e) {
  return {r * q + (r < e ? r : e), q + (r < e ? 1 : 0)};
}

__device__ __forceinline__ float dot2(h2 a, h2 b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// s_waitcnt with vmcnt = VM and the other counters left alone.
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// This wave's LDS accesses done, then a workgroup barrier.  Unlike
// __syncthreads() it does not wait for outstanding global loads, so a ring
// of weight loads stays in flight across it (each later use of a loaded
// register still gets its own vmcnt wait from the compiler).  The empty asm
// statements keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// 3-bit: one 32-row block of one column is three int32 words w0, w1, w2 = the
// 96-bit value V; code i sits at bits 3i..3i+2 of V.  The 32 codes are read
// as 16 fp16 pairs.  Pair P takes a 32-bit window t = V >> src (the words
// themselves, or one shift / funnel shift), code a at bits pa..pa+2 of t
// (low half's mantissa) and code b at bits 16+pb..18+pb (high half's
// mantissa).  Four windows beyond the three words themselves cover all 32
// codes.  Pair table: (src, a, pa, b, pb).
// ---------------------------------------------------------------------------
struct Q3Pair { int src, a, pa, b, pb; };
__host__ __device__ constexpr Q3Pair q3_pair(int i) {
  constexpr Q3Pair t[16] = {
      {0, 0, 0, 6, 2},    {0, 1, 3, 7, 5},    {4, 2, 2, 8, 4},    {4, 3, 5, 9, 7},
      {10, 4, 2, 10, 4},  {10, 5, 5, 11, 7},  {32, 12, 4, 17, 3}, {32, 13, 7, 18, 6},
      {41, 14, 1, 19, 0}, {41, 15, 4, 20, 3}, {41, 16, 7, 21, 6}, {64, 22, 2, 27, 1},
      {64, 23, 5, 28, 4}, {71, 24, 1, 29, 0}, {71, 25, 4, 30, 3}, {71, 26, 7, 31, 6}};
  return t[i];
}

template <int SRC>
__device__ __forceinline__ uint32_t q3_window(uint32_t w0, uint32_t w1, uint32_t w2) {
  if constexpr (SRC == 0) return w0;
  else if constexpr (SRC < 32) return __builtin_amdgcn_alignbit(w1, w0, SRC);
  else if constexpr (SRC == 32) return w1;
  else if constexpr (SRC < 64) return __builtin_amdgcn_alignbit(w2, w1, SRC - 32);
  else if constexpr (SRC == 64) return w2;
  else return w2 >> (SRC - 64);
}

// ---------------------------------------------------------------------------
// Subnormal-pair extractors (the fast path).  Values are in units of 2^-24.
// ---------------------------------------------------------------------------

// int8, stored biased as u = q + 128, in the column-pair layout: byte 0 and
// byte 1 of word w are two consecutive rows of one column, bytes 2 and 3 the
// same rows of the next column.  C selects the column; the result is its two
// rows as (u_lo, u_hi) * 2^-24, one v_perm_b32.
template <int C>
__device__ __forceinline__ uint32_t q8_col_pair(uint32_t w) {
  return __builtin_amdgcn_perm(0u, w, C ? 0x0c030c02u : 0x0c010c00u);
}

// 3-bit: pair P of q3_pair(P) as (c_a * 2^pa, c_b * 2^pb) * 2^-24.
template <int P>
__device__ __forceinline__ h2 q3_pair_sub(uint32_t w0, uint32_t w1, uint32_t w2) {
  constexpr Q3Pair q = q3_pair(P);
  constexpr uint32_t mask = (7u << q.pa) | (7u << (16 + q.pb));
  return as_h2(q3_window<q.src>(w0, w1, w2) & mask);
}

// Accumulation class of a 3-bit pair: the larger of its two mantissa
// offsets.  The activation pair is pre-scaled by (2^(cls-pa), 2^(cls-pb)) so
// both products carry the same factor 2^(cls-24).
__host__ __device__ constexpr int q3_class(int P) {
  return q3_pair(P).pa > q3_pair(P).pb ? q3_pair(P).pa : q3_pair(P).pb;
}
// Classes in use (1, 2, 4, 5, 7) -> accumulator slot 0..4.
__host__ __device__ constexpr int q3_class_slot(int cls) {
  return cls == 1 ? 0 : cls == 2 ? 1 : cls == 4 ? 2 : cls == 5 ? 3 : 4;
}
constexpr int kQ3Classes = 5;
__host__ __device__ constexpr int q3_slot_class(int slot) {
  return slot == 0 ? 1 : slot == 1 ? 2 : slot == 2 ? 4 : slot == 3 ? 5 : 7;
}

template <int P>
__device__ __forceinline__ void q3_block_sub_one(uint32_t w0, uint32_t w1, uint32_t w2, h2* out) {
  out[P] = q3_pair_sub<P>(w0, w1, w2);
}
__device__ __forceinline__ void q3_block_pairs_sub(uint32_t w0, uint32_t w1, uint32_t w2, h2 out[16]) {
  q3_block_sub_one<0>(w0, w1, w2, out);
  q3_block_sub_one<1>(w0, w1, w2, out);
  q3_block_sub_one<2>(w0, w1, w2, out);
  q3_block_sub_one<3>(w0, w1, w2, out);
  q3_block_sub_one<4>(w0, w1, w2, out);
  q3_block_sub_one<5>(w0, w1, w2, out);
  q3_block_sub_one<6>(w0, w1, w2, out);
  q3_block_sub_one<7>(w0, w1, w2, out);
  q3_block_sub_one<8>(w0, w1, w2, out);
  q3_block_sub_one<9>(w0, w1, w2, out);
  q3_block_sub_one<10>(w0, w1, w2, out);
  q3_block_sub_one<11>(w0, w1, w2, out);
  q3_block_sub_one<12>(w0, w1, w2, out);
  q3_block_sub_one<13>(w0, w1, w2, out);
  q3_block_sub_one<14>(w0, w1, w2, out);
  q3_block_sub_one<15>(w0, w1, w2, out);
}

// ---------------------------------------------------------------------------
// Transpose-butterfly reduction over lane bits [LOWBIT, 6) of a wave64.
// Every lane enters with V values; lanes that differ only in those bits hold
// partials of the same V results.  Each step pairs every lane with a partner
// that differs in one lane bit; the lane keeps the half of its values picked
// by that bit and adds the partner's copy of that half, so the work is
// V/2 + V/4 + ... adds instead of V per bit.  On exit value j of a lane is
// result index j + base (bfly_base), summed over all lanes that share the
// lane bits below LOWBIT; lanes whose leftover bits are not zero hold
// duplicates.  No LDS traffic: the partners are reached with
//   bit 5: v_permlane32_swap (lanes l <-> l ^ 32),
//   bit 4: v_permlane16_swap (l <-> l ^ 16),
//   bit 3: DPP row_ror:8     (l <-> l ^ 8 inside a 16-lane row),
//   bit 2: two bank-masked DPP moves, row_shl:4 and row_shr:4 (l <-> l ^ 4),
//   bit 1: DPP quad_perm [2,3,0,1] (l ^ 2),  bit 0: quad_perm [1,0,3,2] (l ^ 1).
// ---------------------------------------------------------------------------
template <int BIT>
__device__ __forceinline__ float bfly_partner(float x) {
  const int xi = __builtin_bit_cast(int, x);
  if constexpr (BIT == 2) {
    // l ^ 4 inside a 16-lane row: banks 0 and 2 (lanes 0-3, 8-11) read l + 4
    // (row_shl:4), banks 1 and 3 read l - 4 (row_shr:4).
    int r = __builtin_amdgcn_update_dpp(0, xi, 0x104, 0xF, 0x5, false);
    r = __builtin_amdgcn_update_dpp(r, xi, 0x114, 0xF, 0xA, false);
    return __builtin_bit_cast(float, r);
  } else {
    // Every lane is written and every source lane exists: bound_ctrl set, so
    // the old value is not needed (no zero-initialising move).
    constexpr int ctrl = BIT == 3 ? 0x128 : BIT == 1 ? 0x4E : 0xB1;
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, xi, ctrl, 0xF, 0xF, true));
  }
}

template <int BIT>
__device__ __forceinline__ float bfly_pair(float lo, float hi, bool upper) {
  if constexpr (BIT == 5 || BIT == 4) {
    // After the swap, each lane's two registers hold its own copy and the
    // partner's copy of the half it keeps.
    const unsigned a = __builtin_bit_cast(unsigned, lo), b = __builtin_bit_cast(unsigned, hi);
    const auto r = BIT == 5 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                            : __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  } else {
    const float mine = upper ? hi : lo, other = upper ? lo : hi;
    return mine + bfly_partner<BIT>(other);
  }
}

template <int V, int BIT, int LOWBIT>
__device__ __forceinline__ void bfly(float* v, int lane) {
  if constexpr (BIT >= LOWBIT) {
    if constexpr (V > 1) {
      const bool upper = (lane >> BIT) & 1;
#pragma unroll
      for (int j = 0; j < V / 2; ++j) v[j] = bfly_pair<BIT>(v[j], v[V / 2 + j], upper);
      bfly<V / 2, BIT - 1, LOWBIT>(v, lane);
    } else {
      if constexpr (BIT == 5 || BIT == 4) {
        v[0] = bfly_pair<BIT>(v[0], v[0], false);
      } else {
        v[0] += bfly_partner<BIT>(v[0]);
      }
      bfly<1, BIT - 1, LOWBIT>(v, lane);
    }
  }
}
// Values left per lane after bfly<V, 5, LOWBIT>.
template <int V, int LOWBIT>
__host__ __device__ constexpr int bfly_left() {
  int v = V;
  for (int b = 5; b >= LOWBIT && v > 1; --b) v /= 2;
  return v;
}
// Result index of a lane's value 0, and whether this lane is the one that
// stores it (its non-transposing reduction bits are zero).
template <int V, int LOWBIT>
__device__ __forceinline__ int bfly_base(int lane, bool& owner) {
  int base = 0, v = V;
  owner = true;
  for (int b = 5; b >= LOWBIT; --b) {
    const int bitv = (lane >> b) & 1;
    if (v > 1) {
      v /= 2;
      base += bitv * v;
    } else if (bitv) {
      owner = false;
    }
  }
  return base;
}

}  // namespace wq
