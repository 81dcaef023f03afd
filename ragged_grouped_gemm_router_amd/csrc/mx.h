// MX (microscaling) FP8 helpers: E4M3 elements with one E8M0 scale per 32
// consecutive elements, following the OCP Microscaling v1.0 format (the
// pages only name "MXFP8"; this is the public definition of that format).
//
//   X     = floor(log2(amax)) - 8 (8 = largest E4M3 exponent), clamped to
//           [-127, 127]; an all-zero block gets X = -127
//   scale = E8M0 code X + 127
//   q_i   = E4M3 round-to-nearest-even of v_i / 2^X, saturated to +-448
#pragma once

#include "common.h"

namespace moe {

// Byte of the E8M0 code of 32-block `blk` (columns 32 blk .. 32 blk + 31)
// of row r, in the scale array of an MX operand with R rows: the codes are
// grouped by 128-column span, [cols/128][R][4], so that one span's four
// codes of a row are one aligned word and consecutive rows' words are
// contiguous (a GEMM k-tile of 128 columns reads the scales of 32
// consecutive rows as one 128-byte line).
__host__ __device__ inline long mx_scale_index(long r, long blk, long R) {
  return ((blk >> 2) * R + r) * 4 + (blk & 3);
}

// E8M0 exponent X of a block from its largest magnitude (fp32).
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xff);
  if (e == 0) return -127;  // zero or fp32-subnormal: floor(log2) <= -127
  return max(e - 127 - 8, -127);
}

// 2^-X as fp32 (X in [-127, 127]; 2^127 is representable).
__device__ __forceinline__ float mx_inv_scale(int X) {
  const int e = 127 - X;  // biased exponent of 2^-X, in [0, 254]
  return e > 0 ? __uint_as_float((uint32_t)e << 23) : __uint_as_float(0x00400000u);
}

// E4M3 (e4m3fn) code of v, rounded to nearest even and saturated to 448.
// Normal E4M3 values have 3 mantissa bits; below 2^-6 the spacing is the
// subnormal step 2^-9. v must be finite.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  uint32_t code;
  if (a >= 0x43e00000u) {             // |v| >= 448
    code = 0x7eu;
  } else if (a < 0x3c800000u) {       // |v| < 2^-6: multiples of 2^-9
    code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // 0..8
  } else {
    uint32_t e = (a >> 23) - 127 + 7;  // 1..15
    uint32_t m = (a >> 20) & 7;
    const uint32_t rest = a & 0xfffffu;
    if (rest > 0x80000u || (rest == 0x80000u && (m & 1))) {
      if (++m == 8) { m = 0; ++e; }
    }
    code = (e << 3) | m;
    if (code > 0x7eu) code = 0x7eu;
  }
  return sign | code;
}

}  // namespace moe
