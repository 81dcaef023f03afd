// MXFP8 quantisation kernels: a bf16 matrix along its rows (weights, once),
// and the permute step's row scatter fused with quantisation of x.
#include "launch.h"
#include "mx.h"

namespace moe {
namespace {

// Quantise 32 values into 32 E4M3 codes packed in q[8] (4 per word,
// lowest index first); returns the E8M0 scale code.
__device__ __forceinline__ uint32_t quant32v(const float (&v)[32],
                                             uint32_t q[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mx_block_exponent(amax);
  const float inv = mx_inv_scale(X);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) word |= e4m3_encode(v[w * 4 + i] * inv) << (8 * i);
    q[w] = word;
  }
  return (uint32_t)(X + 127);
}

// The same for 32 consecutive bf16 values (64 bytes at src, 16-byte
// aligned).
__device__ __forceinline__ uint32_t quant32(const bf16* src, uint32_t q[8]) {
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 x = *(const bf16x8*)(src + c * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[c * 8 + i] = (float)x[i];
  }
  return quant32v(v, q);
}

// Value of an E4M3 (e4m3fn) code: exponent bias 7, 3 mantissa bits,
// subnormals m * 2^-9 (the saturating encoder never writes the NaN code).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? (float)m * 0x1p-9f
                           : __uint_as_float((e + 120u) << 23) * (1.0f + (float)m * 0.125f);
  return (c & 0x80u) ? -mag : mag;
}

// Scale arrays below are in the span-grouped MX layout (mx_scale_index).
//
// The four scale codes of a 128-column span as one word, in the lane
// holding the span's first block (bpr % 4 == 0, so the four blocks of a
// span sit in four consecutive threads, all of them active or none: a
// launch's thread count is a multiple of 4). Lanes of other blocks get 0.
__device__ __forceinline__ uint32_t span_word(uint32_t code) {
  const uint32_t c1 = __shfl_down(code, 1), c2 = __shfl_down(code, 2),
                 c3 = __shfl_down(code, 3);
  return code | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Strided form: block b of 32 is row b / bpr, block b % bpr of a
// contiguous [rows, bpr * 32] source; codes go to q + row * ldq, scales to
// the scale array of a `rows`-row operand, both already offset to the
// first column (a multiple of 128 columns).
__global__ __launch_bounds__(256) void quantize_rows_strided_kernel(
    const bf16* __restrict__ src, long nblk, int bpr, uint8_t* __restrict__ q,
    long ldq, uint8_t* __restrict__ scales) {
  const long b = blockIdx.x * 256L + threadIdx.x;
  if (b >= nblk) return;
  const long r = b / bpr;
  const int blk = (int)(b % bpr);
  uint32_t w[8];
  const uint32_t code = span_word(quant32(src + b * 32, w));
  u32x4* dst = (u32x4*)(q + r * ldq + blk * 32);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  if ((blk & 3) == 0)
    *(uint32_t*)(scales + mx_scale_index(r, blk, nblk / bpr)) = code;
}

// MX codes [rows, cols] with their scales (bpr = cols / 32 per row) back
// to bf16, one thread per 32-block (exact: an E4M3 value times a power of
// two fits bf16's 8-bit mantissa).
__global__ __launch_bounds__(256) void dequantize_rows_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ scales,
    long nblk, int bpr, bf16* __restrict__ out) {
  const long b = blockIdx.x * 256L + threadIdx.x;
  if (b >= nblk) return;
  const float sc =
      ldexpf(1.0f, (int)scales[mx_scale_index(b / bpr, b % bpr, nblk / bpr)] - 127);
  const u32x4* src = (const u32x4*)(q + b * 32);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 w = src[h];
    bf16x8 o[2];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      o[i / 8][i % 8] = (bf16)(e4m3_decode((w[i / 4] >> (8 * (i % 4))) & 0xffu) * sc);
    *(bf16x8*)(out + b * 32 + h * 16) = o[0];
    *(bf16x8*)(out + b * 32 + h * 16 + 8) = o[1];
  }
}

// Transposing quantisation: batch b of a [R, C] bf16 source becomes
// [C, ldq] codes with element (c, r) = Q(src[r][c]), in 32-blocks along r;
// the scales are those of the stacked [batch * C, ldq] operand, from its
// first column's 128-column span (q and scales already offset there). A workgroup stages a 32 x 64
// tile in LDS; thread c < 64 then quantises column c's 32 values. (Used
// once per weight set.)
__global__ __launch_bounds__(256) void quantize_cols_kernel(
    const bf16* __restrict__ src, int R, int C, uint8_t* __restrict__ q,
    long ldq, long q_bstride, uint8_t* __restrict__ scales) {
  __shared__ float tile[32][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 32, b = blockIdx.z;
  const bf16* sb = src + (long)b * R * C;
  {
    const int r = threadIdx.x / 8, c = (threadIdx.x % 8) * 8;
    const bf16x8 x = *(const bf16x8*)(sb + (long)(r0 + r) * C + c0 + c);
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[r][c + i] = (float)x[i];
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int c = threadIdx.x;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = tile[i][c];
  uint32_t w[8];
  const uint32_t code = quant32v(v, w);
  u32x4* dst = (u32x4*)(q + b * q_bstride + (long)(c0 + c) * ldq + r0);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  scales[mx_scale_index((long)b * C + c0 + c, r0 / 32, (long)gridDim.z * C)] =
      (uint8_t)code;
}

__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const bf16* __restrict__ src, long nblk, int bpr, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales) {
  // (codes stay in row order; one thread writes one block's scale byte)
  const long b = blockIdx.x * 256L + threadIdx.x;
  if (b >= nblk) return;
  uint32_t w[8];
  const uint32_t code = span_word(quant32(src + b * 32, w));
  u32x4* dst = (u32x4*)(q + b * 32);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  if ((b & 3) == 0)
    *(uint32_t*)(scales + mx_scale_index(b / bpr, b % bpr, nblk / bpr)) = code;
}

// one thread per (token, 32-block): quantise once, write to the token's K
// sorted slots (scales of the n / bpr * K-row x_perm)
__global__ __launch_bounds__(256) void scatter_rows_mxfp8_kernel(
    const bf16* __restrict__ x, long n, int K, int bpr,
    const int32_t* __restrict__ dest, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i >= n) return;
  const long t = i / bpr;
  const int blk = (int)(i % bpr);
  uint32_t w[8];
  const uint32_t code = span_word(quant32(x + t * bpr * 32 + blk * 32, w));
  for (int k = 0; k < K; ++k) {
    const long p = dest[t * K + k];
    u32x4* dst = (u32x4*)(xq + (p * bpr + blk) * 32);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    if ((blk & 3) == 0)
      *(uint32_t*)(xs + mx_scale_index(p, blk, n / bpr * K)) = code;
  }
}

}  // namespace

hipError_t launch_quantize_mxfp8(const void* src, long rows, long cols,
                                 uint8_t* q, uint8_t* scales, hipStream_t s) {
  const long nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)((nblk + 255) / 256)),
                     dim3(256), 0, s, (const bf16*)src, nblk, (int)(cols / 32),
                     q, scales);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_strided(const void* src, long rows,
                                         long cols, uint8_t* q, long ldq,
                                         uint8_t* scales, hipStream_t s) {
  const long nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_rows_strided_kernel,
                     dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s,
                     (const bf16*)src, nblk, (int)(cols / 32), q, ldq, scales);
  return hipGetLastError();
}

hipError_t launch_dequantize_mxfp8(const uint8_t* q, const uint8_t* scales,
                                   long rows, long cols, void* out,
                                   hipStream_t s) {
  const long nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(dequantize_rows_kernel,
                     dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, q,
                     scales, nblk, (int)(cols / 32), (bf16*)out);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_cols(const void* src, long batch, int R,
                                      int C, uint8_t* q, long ldq,
                                      uint8_t* scales, hipStream_t s) {
  if (batch == 0 || R == 0 || C == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_cols_kernel,
                     dim3((unsigned)(C / 64), (unsigned)(R / 32),
                          (unsigned)batch),
                     dim3(256), 0, s, (const bf16*)src, R, C, q, ldq,
                     (long)C * ldq, scales);
  return hipGetLastError();
}

hipError_t launch_scatter_rows_mxfp8(const void* x, int T, int K, int d,
                                     const int32_t* dest, uint8_t* xq,
                                     uint8_t* xs, hipStream_t s) {
  const int bpr = d / 32;
  const long n = (long)T * bpr;
  hipLaunchKernelGGL(scatter_rows_mxfp8_kernel,
                     dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const bf16*)x, n, K, bpr, dest, xq, xs);
  return hipGetLastError();
}

}  // namespace moe
