// Shared pieces of the 4-bit (and 2-bit) packed layout: panel and block
// sizes, and the conversion of a packed word into a matrix-core operand.
//
// A panel is 16 output columns; its rows, in group order, are cut into blocks
// of 128 (4-bit) or 256 (2-bit) rows.  Block (panel p, block b) is 1 KB:
// lane l owns 16 bytes = 4 words, word j holding the 8 codes of column
// 16 p + l % 16, rows 128 b + 32 j + 8 (l / 16) .. +7, row +e in nibble e:
// the B operand of MFMA step j of the block.
#pragma once

#include "wq_device.hpp"

namespace wq {

constexpr int kQ4Panel = 16;   // columns per panel (one MFMA tile)
constexpr int kQ4Block = 128;  // rows per 4-bit block (4 MFMA steps of 32)
// Rows per 1 KB block: 128 four-bit or 256 two-bit codes per 16 columns.
template <int BITS>
constexpr int block_rows() { return BITS == 4 ? 128 : 256; }

// The four code pairs (e, e + 4), e = 0..3, of one word as one MFMA operand:
// each half an fp16 subnormal whose mantissa is the code, i.e. u * 2^-24.
// The 8 rows of the word enter in the order 0 4 1 5 2 6 3 7.
__device__ __forceinline__ u32x4 q4_mfma_operand(uint32_t w) {
  return u32x4{w & 0x000F000Fu, (w >> 4) & 0x000F000Fu, (w >> 8) & 0x000F000Fu,
               (w >> 12) & 0x000F000Fu};
}

// Position of row e (0..7) of an octet among the 8 halves of an operand
// (the order above).
__host__ __device__ constexpr int q4_pos(int e) { return 2 * (e & 3) + (e >> 2); }

}  // namespace wq
