// Expert histogram, prefix scan, stable permutation, row scatter, and the
// gate-weighted combine (forward and backward).
//
// Counting sort in three passes, no atomics on global memory:
//   1. each workgroup counts its chunk of kPermChunk copies into an LDS
//      histogram and writes it as column b of block_hist[E, nblk];
//   2. one workgroup turns block_hist into per-(expert, chunk) starting
//      slots: an exclusive scan over chunks per expert, plus the expert's
//      offset from an exclusive scan over experts; it also publishes the
//      expert offsets and the row-tile prefix for each GEMM tile height;
//   3. one wavefront per chunk walks its copies in order, 64 at a time;
//      lanes with the same expert find each other with log2(E) ballots,
//      rank among themselves by popcount, and the last of them advances
//      the expert's running slot in LDS. Order within an expert therefore
//      follows the copy index j = t*K + k, which makes the sort stable.
#include "gemm.h"
#include "launch.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx,
                                                   int TK, int E,
                                                   int32_t* __restrict__ block_hist,
                                                   int nblk) {
  __shared__ int32_t h[MOE_E_MAX];
  for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const int j_end = min(TK, (b + 1) * kPermChunk);
  for (int j = b * kPermChunk + threadIdx.x; j < j_end; j += 256)
    atomicAdd(&h[idx[j]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) block_hist[(long)e * nblk + b] = h[e];
}

// Exclusive scan of one value per thread over a 1024-thread block.
__device__ int block_exclusive_scan(int v, int32_t (*buf)[1024]) {
  const int tid = threadIdx.x;
  int pin = 0;
  buf[0][tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int x = buf[pin][tid];
    if (tid >= off) x += buf[pin][tid - off];
    buf[pin ^ 1][tid] = x;
    pin ^= 1;
    __syncthreads();
  }
  const int incl = buf[pin][tid];
  __syncthreads();
  return incl - v;
}

struct TileOffPtrs { int32_t* p[kNumTileBM]; };

__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ block_hist,
                                                    int nblk, int E,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    TileOffPtrs toff) {
  __shared__ int32_t buf[2][1024];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    int32_t* row = block_hist + (long)e * nblk;
    for (int b = 0; b < nblk; ++b) {
      const int v = row[b];
      row[b] = total;
      total += v;
    }
  }
  const int excl = block_exclusive_scan(total, buf);
  if (e < E) {
    counts[e] = total;
    offsets[e] = excl;
    int32_t* row = block_hist + (long)e * nblk;
    for (int b = 0; b < nblk; ++b) row[b] += excl;
  }
  if (e == E - 1) offsets[E] = excl + total;
#pragma unroll
  for (int s = 0; s < kNumTileBM; ++s) {
    const int bm = kTileBM[s];
    const int tiles = e < E ? (total + bm - 1) / bm : 0;
    const int tx = block_exclusive_scan(tiles, buf);
    if (e < E) toff.p[s][e] = tx;
    if (e == E - 1) toff.p[s][E] = tx + tiles;
  }
}

// Row-tile prefix for every tile height from the expert offsets alone.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets,
                                                           int E, TileOffPtrs toff) {
  __shared__ int32_t buf[2][1024];
  const int e = threadIdx.x;
  const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
#pragma unroll
  for (int s = 0; s < kNumTileBM; ++s) {
    const int bm = kTileBM[s];
    const int tiles = (cnt + bm - 1) / bm;
    const int tx = block_exclusive_scan(tiles, buf);
    if (e < E) toff.p[s][e] = tx;
    if (e == E - 1) toff.p[s][E] = tx + tiles;
  }
}

__global__ __launch_bounds__(kWave) void rank_kernel(const int32_t* __restrict__ idx,
                                                     int TK, int E, int nbits,
                                                     const int32_t* __restrict__ block_hist,
                                                     int nblk,
                                                     int32_t* __restrict__ sorted_src,
                                                     int32_t* __restrict__ dest) {
  __shared__ int32_t run[MOE_E_MAX];
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += kWave) run[e] = block_hist[(long)e * nblk + b];
  __syncthreads();
  const int j_end = min(TK, (b + 1) * kPermChunk);
  for (int j0 = b * kPermChunk; j0 < j_end; j0 += kWave) {
    const int j = j0 + lane;
    const bool valid = j < j_end;
    const int e = valid ? idx[j] : 0;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bal = __ballot(valid && on);
      m &= on ? bal : ~bal;
    }
    if (valid) {
      const int base = run[e];
      const int p = base + __popcll(m & ((1ull << lane) - 1ull));
      dest[j] = p;
      sorted_src[p] = j;
      if ((m >> lane) == 1ull) run[e] = base + __popcll(m);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void scatter_rows_kernel(const u32x4* __restrict__ x,
                                                           long n, int K, int cpr,
                                                           const int32_t* __restrict__ dest,
                                                           u32x4* __restrict__ xp) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i >= n) return;
  const long t = i / cpr;
  const int c = (int)(i % cpr);
  const u32x4 v = x[i];
  for (int k = 0; k < K; ++k) xp[(long)dest[t * K + k] * cpr + c] = v;
}

// 8 consecutive elements <-> fp32
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 a = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
  *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = (bf16)v[i];
  *(bf16x8*)p = a;
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y,
                                                      const int32_t* __restrict__ dest,
                                                      const float* __restrict__ w,
                                                      const T* __restrict__ add,
                                                      T* __restrict__ out, long n,
                                                      int K, int d) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i >= n) return;
  const int cpr = d / 8;
  const long t = i / cpr;
  const int c = (int)(i % cpr) * 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int k = 0; k < K; ++k) {
    const long p = dest[t * K + k];
    const float wk = w ? w[t * K + k] : 1.0f;
    float v[8];
    load8(y + p * d + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = fmaf(wk, v[q], acc[q]);
  }
  if (add) {
    float v[8];
    load8(add + t * d + c, v);
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += v[q];
  }
  store8(out + t * d + c, acc);
}

template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy,
                                                          const T* __restrict__ y,
                                                          const int32_t* __restrict__ dest,
                                                          const float* __restrict__ w,
                                                          T* __restrict__ dy_perm,
                                                          float* __restrict__ d_w,
                                                          int K, int d) {
  __shared__ float red[256 / kWave][MOE_K_MAX];
  const long t = blockIdx.x;
  float part[MOE_K_MAX];
#pragma unroll
  for (int k = 0; k < MOE_K_MAX; ++k) part[k] = 0.0f;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float g[8];
    load8(dy + t * d + c, g);
#pragma unroll
    for (int k = 0; k < MOE_K_MAX; ++k) {
      if (k >= K) break;
      const long p = dest[t * K + k];
      const float wk = w[t * K + k];
      float v[8], o[8];
      load8(y + p * d + c, v);
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        s = fmaf(g[q], v[q], s);
        o[q] = wk * g[q];
      }
      part[k] += s;
      store8(dy_perm + p * d + c, o);
    }
  }
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
#pragma unroll
  for (int k = 0; k < MOE_K_MAX; ++k) {
    if (k >= K) break;
    float v = part[k];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) red[wv][k] = v;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < 256 / kWave; ++q) s += red[q][threadIdx.x];
    d_w[t * K + threadIdx.x] = s;
  }
}

}  // namespace

hipError_t launch_histogram_scan(const int32_t* idx, int TK, int E,
                                 int32_t* block_hist, int32_t* counts,
                                 int32_t* offsets, int32_t* const* tile_off,
                                 hipStream_t s) {
  const int nblk = (TK + kPermChunk - 1) / kPermChunk;
  hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(256), 0, s, idx, TK, E,
                     block_hist, nblk);
  TileOffPtrs tp;
  for (int i = 0; i < kNumTileBM; ++i) tp.p[i] = tile_off[i];
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, block_hist, nblk,
                     E, counts, offsets, tp);
  return hipGetLastError();
}

hipError_t launch_tile_prefix(const int32_t* offsets, int E,
                              int32_t* const* tile_off, hipStream_t s) {
  TileOffPtrs tp;
  for (int i = 0; i < kNumTileBM; ++i) tp.p[i] = tile_off[i];
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, E, tp);
  return hipGetLastError();
}

hipError_t launch_rank(const int32_t* idx, int TK, int E,
                       const int32_t* block_hist, int32_t* sorted_src,
                       int32_t* dest, hipStream_t s) {
  const int nblk = (TK + kPermChunk - 1) / kPermChunk;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  hipLaunchKernelGGL(rank_kernel, dim3(nblk), dim3(kWave), 0, s, idx, TK, E,
                     nbits, block_hist, nblk, sorted_src, dest);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const void* x, int T, int K, long row_bytes,
                               const int32_t* dest, void* x_perm,
                               hipStream_t s) {
  const int cpr = (int)(row_bytes / 16);
  const long n = (long)T * cpr;
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, s, (const u32x4*)x, n, K, cpr, dest,
                     (u32x4*)x_perm);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* y, const int32_t* dest,
                          const float* w, const void* add, void* out, int T,
                          int K, int d, hipStream_t s) {
  const long n = (long)T * (d / 8);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, s, (const float*)y,
                       dest, w, (const float*)add, (float*)out, n, K, d);
  else
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, block, 0, s, (const bf16*)y,
                       dest, w, (const bf16*)add, (bf16*)out, n, K, d);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(int dtype, const void* dy, const void* y,
                              const int32_t* dest, const float* w,
                              void* dy_perm, float* d_w, int T, int K, int d,
                              hipStream_t s) {
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(combine_bwd_kernel<float>, dim3(T), dim3(256), 0, s,
                       (const float*)dy, (const float*)y, dest, w,
                       (float*)dy_perm, d_w, K, d);
  else
    hipLaunchKernelGGL(combine_bwd_kernel<bf16>, dim3(T), dim3(256), 0, s,
                       (const bf16*)dy, (const bf16*)y, dest, w, (bf16*)dy_perm,
                       d_w, K, d);
  return hipGetLastError();
}

}  // namespace moe
