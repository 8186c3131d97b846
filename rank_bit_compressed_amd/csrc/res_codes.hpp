// res_codes.hpp -- the 2-bit rotated residual's codes in the matrix and vector units (gfx950), shared by the
// kernels that add it: the per-head INT4 residual kernel and the block-shared kernel.
#pragma once

#include "kvc_common.hpp"

namespace kvc {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// fp8 (e4m3) x fp8 32x32x64 product, fp32 accumulate; A unscaled, B scaled by 2^9 (E8M0 exponents 127, 136): a
// residual code c stored alone in a byte is the e4m3 pattern of c * 2^-9, so B reads as the integer c
__device__ inline f32x16_t mfma_f8_codes(v8i_t a, v8i_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 136);
}
// Coordinate (within a 64-coordinate block) of byte b of lane half hf's key residual operand: byte q of dword o is
// code m + 4q (m = o % 4) of the block's code dword 2hf + o / 4.
__host__ __device__ constexpr int res8_coord(int hf, int b) {
  return 16 * (2 * hf + (b >> 4)) + ((b >> 2) & 3) + 4 * (b & 3);
}

// Eight 2-bit residual codes c of a code dword x (code k at bits 2k) as exact fp16 2c - 3 for lane half hf:
// element e is code 4hf + e / 2 + 8 (e % 2).  In xs = x >> 8hf, codes 4hf + kk and 4hf + kk + 8 sit at bits 2kk
// and 2kk + 16; one shift (left by one for kk = 0, right by 2kk - 1 otherwise) and a mask and an or put them
// into the mantissas of two fp16 1024s (1024 + 2c, exact), and subtracting 1027 leaves 2c - 3.  Bit operations
// and one packed subtraction per pair: the fp8 and permute conversions issue at about a third of their rate.
__device__ inline h8 res_2c3(uint32_t x, int hf) {
  const uint32_t xs = x >> (8 * hf);
  const h2 off = {(_Float16)1027.0f, (_Float16)1027.0f};
  h8 r;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const uint32_t sh = kk == 0 ? xs << 1 : xs >> (2 * kk - 1);
    const uint32_t y = (sh & 0x00060006u) | 0x64006400u;
    const h2 v = as_h2(y) - off;
    r[2 * kk] = v.x;
    r[2 * kk + 1] = v.y;
  }
  return r;
}
__device__ inline int res_coord(int hf, int e) { return 4 * hf + (e >> 1) + 8 * (e & 1); }


}  // namespace kvc
