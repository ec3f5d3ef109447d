// fp4 (e2m1) sign planes of the packed codes, shared by the decode GEMVs that read them on the
// scaled matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// Sources: zhichai.net reading note, "Step 2" dequantization and "Industry implications:
// multiplication-free inference" (B_re, B_im in {-1, 0, 1}).
//
// With u = B_re + B_im and v = B_re - B_im every codeword gives u, v in {+1, -1}: code 0 (+1)
// u = v = +1; code 1 (+i) u = +1, v = -1; code 2 (-1) u = v = -1; code 3 (-i) u = -1, v = +1.
// The planes are held as +-6, the fp4 value whose nibble is 0b s111, so setting the low three
// bits of every nibble turns a sign bit into an operand.  In a 256-column chunk lane l = 16g + r of
// a wave holds row r, columns 64g .. 64g + 63 of the tile (four packed words); MFMA step s < 2
// takes words 2s and 2s + 1, so its A operand covers columns 64g + 32s .. 64g + 32s + 31 in the
// element order f4_column gives.
#pragma once

#include "common.hpp"

namespace f2i {

typedef int v8i __attribute__((ext_vector_type(8)));

// Column (within its 256-column chunk) of element q < 32 of the fp4 plane of lane group g at MFMA
// step s: word 2s + q/16 of the lane's four words; in that word, the upper (h = 1) or lower
// (h = 0) code of nibble j.  Code p of a word sits in bits 8(p % 4) + 2(p / 4), so nibble j holds
// codes p = 4(2(j % 2)) + j/2 (lower) and p + 4 (upper).
__host__ __device__ __forceinline__ int f4_column(int g, int s, int q) {
  const int wd = 2 * s + (q >> 4), h = (q >> 3) & 1, j = q & 7;
  return 64 * g + 16 * wd + 4 * (2 * (j & 1) + h) + (j >> 1);
}

constexpr uint32_t kLow3 = 0x77777777u;     // the non-sign bits of every nibble: fp4 +-6

// u and v planes (fp4 +-6) of one packed word: [lower halves, upper halves] of its nibbles.
__device__ __forceinline__ void decode_f4_word(uint32_t w, uint32_t& u_lo, uint32_t& u_hi,
                                               uint32_t& v_lo, uint32_t& v_hi) {
  const uint32_t w1 = w << 1;
  u_hi = w | kLow3;
  u_lo = (w << 2) | kLow3;                                    // v_lshl_or_b32
  v_hi = __builtin_amdgcn_bitop3_b32(w, w1, kLow3, 0xBE);     // (w ^ w1) | kLow3
  v_lo = ((w ^ w1) << 2) | kLow3;
}

__device__ __forceinline__ void decode_f4(uint32_t w0, uint32_t w1, v8i& u, v8i& v) {
  uint32_t a0, a1, b0, b1, c0, c1, d0, d1;
  decode_f4_word(w0, a0, a1, c0, c1);
  decode_f4_word(w1, b0, b1, d0, d1);
  u = v8i{(int)a0, (int)a1, (int)b0, (int)b1, 0, 0, 0, 0};
  v = v8i{(int)c0, (int)c1, (int)d0, (int)d1, 0, 0, 0, 0};
}

}  // namespace f2i
