// MXFP8 quantisation kernels: a bf16 matrix along its rows (weights, once),
// and the permute step's row scatter fused with quantisation of x.
#include "launch.h"
#include "mx.h"

namespace moe {
namespace {

// Quantise 32 consecutive bf16 values (64 bytes at src, 16-byte aligned)
// into 32 E4M3 codes packed in q[8] (4 per word, lowest address first);
// returns the E8M0 scale code.
__device__ __forceinline__ uint32_t quant32(const bf16* src, uint32_t q[8]) {
  float v[32];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 x = *(const bf16x8*)(src + c * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[c * 8 + i] = (float)x[i];
  }
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

__global__ __launch_bounds__(256) void quantize_rows_kernel(
    const bf16* __restrict__ src, long nblk, int bpr, uint8_t* __restrict__ q,
    uint8_t* __restrict__ scales) {
  const long b = blockIdx.x * 256L + threadIdx.x;
  if (b >= nblk) return;
  uint32_t w[8];
  const uint32_t code = quant32(src + b * 32, w);
  u32x4* dst = (u32x4*)(q + b * 32);
  dst[0] = u32x4{w[0], w[1], w[2], w[3]};
  dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  scales[b] = (uint8_t)code;
  (void)bpr;
}

// one thread per (token, 32-block): quantise once, write to the token's K
// sorted slots
__global__ __launch_bounds__(256) void scatter_rows_mxfp8_kernel(
    const bf16* __restrict__ x, long n, int K, int bpr,
    const int32_t* __restrict__ dest, uint8_t* __restrict__ xq,
    uint8_t* __restrict__ xs) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i >= n) return;
  const long t = i / bpr;
  const int blk = (int)(i % bpr);
  uint32_t w[8];
  const uint32_t code = quant32(x + t * bpr * 32 + blk * 32, w);
  for (int k = 0; k < K; ++k) {
    const long p = dest[t * K + k];
    u32x4* dst = (u32x4*)(xq + (p * bpr + blk) * 32);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    xs[p * bpr + blk] = (uint8_t)code;
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
