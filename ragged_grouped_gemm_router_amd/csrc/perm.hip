// Expert histogram, prefix scan, stable permutation, row scatter, and the
// gate-weighted combine (forward and backward).
//
// Counting sort in three kernels, no atomics on global memory:
//   1. hist_rank: each workgroup takes a chunk of kPermChunk copies (copy
//      j = t*K + k); each of its four waves walks its quarter in order, 64
//      copies at a time, finds the lanes holding the same expert with
//      log2(E) ballots and ranks them by popcount against a per-wave LDS
//      count. A prefix over the four waves then gives every copy its rank
//      among the chunk's copies of its expert, in copy order, and the
//      chunk's histogram is written as row b of block_hist[nblk, E];
//   2. scan: one workgroup; a few threads per expert each sum a range of
//      chunks, and one exclusive scan over all (expert, range) pairs gives
//      each range its first slot. block_hist becomes, in place, the first
//      slot of every (chunk, expert); counts, offsets and the row-tile
//      prefix of every GEMM tile height are written too;
//   3. scatter: slot of copy j = block_hist[j / kPermChunk, e] + its rank.
//      Each workgroup writes dest and sorted_src for its tokens' copies,
//      then copies their rows, reading each row of x once.
// The order within an expert follows the copy index, so the sort is stable.
#include "gemm.h"
#include "launch.h"
#include "rank.h"

namespace moe {
namespace {

constexpr int kRankWaves = 4;

__global__ __launch_bounds__(kRankWaves * kWave) void hist_rank_kernel(
    const int32_t* __restrict__ idx, int TK, int E, int nbits,
    int32_t* __restrict__ block_hist, int32_t* __restrict__ rank) {
  __shared__ int32_t cnt[kRankWaves][MOE_E_MAX];
  const long j0 = (long)blockIdx.x * kPermChunk;
  const int n = (int)min((long)kPermChunk, TK - j0);
  rank_chunk<kRankWaves, MOE_E_MAX>([&](int i) { return idx[j0 + i]; }, n, E,
                                    nbits, j0, cnt,
                                    block_hist + (long)blockIdx.x * E, rank);
}

// Exclusive scan over a block of NW waves (1024 threads by default) of N
// values per thread at once (v[i] of thread t scanned across threads): an
// inclusive scan inside each wave by shuffles, then one pass over the NW
// wave totals. wsum holds 16 * N ints of LDS.
template <int N, int NW = 16>
__device__ void block_exclusive_scan(int (&v)[N], int32_t* wsum) {
  static_assert(NW <= 16, "wave totals");
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  int x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = v[i];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int y = __shfl_up(x[i], off);
      if (lane >= off) x[i] += y;
    }
  }
  if (lane == kWave - 1)
#pragma unroll
    for (int i = 0; i < N; ++i) wsum[i * 16 + wv] = x[i];
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      int s = lane < NW ? wsum[i * 16 + lane] : 0;
      const int own = s;
#pragma unroll
      for (int off = 1; off < NW; off <<= 1) {
        const int y = __shfl_up(s, off);
        if (lane >= off) s += y;
      }
      if (lane < NW) wsum[i * 16 + lane] = s - own;  // exclusive wave base
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = x[i] - v[i] + wsum[i * 16 + wv];
  __syncthreads();
}

struct TileOffPtrs { int32_t* p[kNumTileBM]; };

// Row-tile prefix of every tile height, from expert counts (thread e of a
// block of NW waves, E <= 64 * NW).
template <int NW = 16>
__device__ void write_tile_prefix(int cnt, int E, const TileOffPtrs& toff,
                                  int32_t* wsum) {
  const int e = threadIdx.x;
  int tiles[kNumTileBM], tx[kNumTileBM];
#pragma unroll
  for (int s = 0; s < kNumTileBM; ++s) {
    tiles[s] = e < E ? (cnt + kTileBM[s] - 1) / kTileBM[s] : 0;
    tx[s] = tiles[s];
  }
  block_exclusive_scan<kNumTileBM, NW>(tx, wsum);
#pragma unroll
  for (int s = 0; s < kNumTileBM; ++s) {
    if (e < E) toff.p[s][e] = tx[s];
    if (e == E - 1) toff.p[s][E] = tx[s] + tiles[s];
  }
}

// block_hist[nblk, E] of counts -> first slot of each (chunk, expert).
// Thread tid = e * tpe + sub sums chunks [sub * cps, ...) of expert e; the
// block scan in that (expert-major) order yields the range's first slot.
__global__ __launch_bounds__(1024) void scan_kernel(int32_t* __restrict__ block_hist,
                                                    int nblk, int E, int tpe,
                                                    int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets,
                                                    TileOffPtrs toff) {
  __shared__ int32_t wsum[16 * kNumTileBM];
  __shared__ int32_t first[MOE_E_MAX], cnt_s[MOE_E_MAX];
  const int tid = threadIdx.x;
  const int e = tid / tpe, sub = tid % tpe;
  const int cps = (nblk + tpe - 1) / tpe;
  const int b0 = min(nblk, sub * cps), b1 = min(nblk, b0 + cps);
  // 8 chunks per step, loads first, so their latencies overlap
  constexpr int U = 8;
  int sum = 0;
  if (e < E)
    for (int b = b0; b < b1; b += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = b + u < b1 ? block_hist[(long)(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) sum += v[u];
    }
  int ex[1] = {sum};
  block_exclusive_scan(ex, wsum);
  const int excl = ex[0];
  if (e < E) {
    int run = excl;
    for (int b = b0; b < b1; b += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        v[u] = b + u < b1 ? block_hist[(long)(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b + u < b1) block_hist[(long)(b + u) * E + e] = run;
        run += v[u];
      }
    }
    if (sub == 0) {
      first[e] = excl;
      offsets[e] = excl;
    }
  }
  if (tid == 1023) offsets[E] = excl + sum;  // total copies
  __syncthreads();
  if (e < E && sub == tpe - 1) cnt_s[e] = excl + sum - first[e];
  __syncthreads();
  const int cnt = tid < E ? cnt_s[tid] : 0;
  if (tid < E) counts[tid] = cnt;
  write_tile_prefix(cnt, E, toff, wsum);
}

// Row-tile prefix for every tile height from the expert offsets alone.
__global__ __launch_bounds__(1024) void tile_prefix_kernel(const int32_t* __restrict__ offsets,
                                                           int E, TileOffPtrs toff) {
  __shared__ int32_t wsum[16 * kNumTileBM];
  const int e = threadIdx.x;
  const int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
  write_tile_prefix(cnt, E, toff, wsum);
}

// Slots of this workgroup's copies (tokens [t0, t0 + tpb)) into LDS, and
// dest / sorted_src for them. Returns the number of copies.
__device__ __forceinline__ int block_slots(const int32_t* __restrict__ idx,
                                           const int32_t* __restrict__ first,
                                           const int32_t* __restrict__ rank,
                                           int E, int K, long t0, int tpb, int T,
                                           int32_t* __restrict__ dest,
                                           int32_t* __restrict__ sorted_src,
                                           int32_t* slot) {
  const int ntok = (int)min((long)tpb, T - t0);
  const int n = ntok * K;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const long j = t0 * K + i;
    const int p = first[(j / kPermChunk) * E + idx[j]] + rank[j];
    slot[i] = p;
    dest[j] = p;
    sorted_src[p] = (int)j;
  }
  __syncthreads();
  return ntok;
}

constexpr int kScatterThreads = 256;

__global__ __launch_bounds__(256) void slots_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ first,
    const int32_t* __restrict__ rank, long TK, int E,
    int32_t* __restrict__ dest, int32_t* __restrict__ sorted_src) {
  const long j = blockIdx.x * 256L + threadIdx.x;
  if (j >= TK) return;
  const int p = first[(j / kPermChunk) * E + idx[j]] + rank[j];
  dest[j] = p;
  sorted_src[p] = (int)j;
}

// x_perm[slot(t, k)] = x[t] for the workgroup's tpb tokens; cpr 16-byte
// chunks per row.
// SCAN (E * nblk <= kScatterThreads): `first` still holds the chunk
// histograms; every workgroup scans them in LDS (expert-major order, as
// the scan kernel does) instead of a separate single-workgroup launch,
// and workgroup 0 writes counts, offsets and the row-tile prefixes.
template <bool SCAN>
__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(
    const u32x4* __restrict__ x, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ first, const int32_t* __restrict__ rank,
    int T, int E, int K, int cpr, int tpb, int32_t* __restrict__ dest,
    int32_t* __restrict__ sorted_src, u32x4* __restrict__ xp, int nblk,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    TileOffPtrs toff) {
  __shared__ int32_t slot[kScatterThreads];
  __shared__ int32_t sfirst[SCAN ? kScatterThreads : 1];
  __shared__ int32_t wsum[16 * kNumTileBM];
  constexpr int NW = kScatterThreads / kWave;
  const int32_t* fst = first;
  if constexpr (SCAN) {
    const int tid = threadIdx.x, ne = E * nblk;
    const int e = tid / nblk, c = tid % nblk;
    int v[1] = {tid < ne ? first[(long)c * E + e] : 0};
    block_exclusive_scan<1, NW>(v, wsum);
    if (tid < ne) sfirst[c * E + e] = v[0];
    __syncthreads();
    if (blockIdx.x == 0) {
      const int TK = T * K;
      int cnt = 0;
      if (tid < E) {  // chunk 0 of expert e: its first slot
        const int o = sfirst[tid];
        cnt = (tid + 1 < E ? sfirst[tid + 1] : TK) - o;
        counts[tid] = cnt;
        offsets[tid] = o;
      }
      if (tid == 0) offsets[E] = TK;
      write_tile_prefix<NW>(cnt, E, toff, wsum);
    }
    fst = sfirst;
  }
  const long t0 = (long)blockIdx.x * tpb;
  const int ntok = block_slots(idx, fst, rank, E, K, t0, tpb, T, dest,
                               sorted_src, slot);
  const int n = ntok * cpr;
  constexpr int U = 4;  // chunks in flight per thread
  for (int i0 = threadIdx.x; i0 < n; i0 += U * kScatterThreads) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kScatterThreads;
      if (i < n) v[u] = x[(t0 + i / cpr) * cpr + i % cpr];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kScatterThreads;
      if (i < n) {
        const int tl = i / cpr, c = i % cpr;
        for (int k = 0; k < K; ++k) xp[(long)slot[tl * K + k] * cpr + c] = v[u];
      }
    }
  }
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

// out[t] = sum_k w[t,k] * y[dest[t*K+k]] (+ add[t]) for the workgroup's
// tpb tokens, 8 columns per item, fp32 accumulation in k order and one
// rounding; U items per thread keep U*K row loads in flight.
template <typename T, int U>
__global__ __launch_bounds__(kScatterThreads) void combine_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ dest,
    const float* __restrict__ w, const T* __restrict__ add, T* __restrict__ out,
    int Ttok, int K, int d, int tpb) {
  __shared__ int32_t sd[kScatterThreads];
  __shared__ float sw[kScatterThreads];
  const long t0 = (long)blockIdx.x * tpb;
  const int ntok = (int)min((long)tpb, Ttok - t0);
  for (int i = threadIdx.x; i < ntok * K; i += kScatterThreads) {
    sd[i] = dest[t0 * K + i];
    sw[i] = w ? w[t0 * K + i] : 1.0f;
  }
  __syncthreads();
  const int cpr = d / 8, n = ntok * cpr;
  for (int i0 = threadIdx.x; i0 < n; i0 += U * kScatterThreads) {
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kScatterThreads;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
      if (i >= n) continue;
      const int tl = i / cpr, c = (i % cpr) * 8;
      for (int k = 0; k < K; ++k) {
        float v[8];
        load8(y + (long)sd[tl * K + k] * d + c, v);
        const float wk = sw[tl * K + k];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] = fmaf(wk, v[q], acc[u][q]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kScatterThreads;
      if (i >= n) continue;
      const int tl = i / cpr, c = (i % cpr) * 8;
      const long o = (t0 + tl) * d + c;
      if (add) {
        float v[8];
        load8(add + o, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] += v[q];
      }
      store8(out + o, acc[u]);
    }
  }
}

// The same for a compile-time K: the U * KT row loads of a thread's items
// are issued together (indices clamped instead of branched on, so the
// code is straight-line), then summed in k order as above.
template <typename T, int U, int KT>
__global__ __launch_bounds__(kScatterThreads) void combine_k_kernel(
    const T* __restrict__ y, const int32_t* __restrict__ dest,
    const float* __restrict__ w, const T* __restrict__ add, T* __restrict__ out,
    int Ttok, int d, int tpb) {
  __shared__ int32_t sd[kScatterThreads];
  __shared__ float sw[kScatterThreads];
  const long t0 = (long)blockIdx.x * tpb;
  const int ntok = (int)min((long)tpb, Ttok - t0);
  for (int i = threadIdx.x; i < ntok * KT; i += kScatterThreads) {
    sd[i] = dest[t0 * KT + i];
    sw[i] = w ? w[t0 * KT + i] : 1.0f;
  }
  __syncthreads();
  const int cpr = d / 8, n = ntok * cpr;
  for (int i0 = threadIdx.x; i0 < n; i0 += U * kScatterThreads) {
    float v[U][KT][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u * kScatterThreads, n - 1);
      const int tl = i / cpr, c = (i % cpr) * 8;
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const T* row = y + (long)sd[tl * KT + k] * d + c;
        if constexpr (sizeof(T) == 2 && KT >= 8) {
          // many rows gathered per token, each read once: streaming
          // loads (measured: K = 8 combine 126 -> 107 us at d = 7168)
          const bf16x8 a = __builtin_nontemporal_load((const bf16x8*)row);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[u][k][q] = (float)a[q];
        } else {
          load8(row, v[u][k]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kScatterThreads;
      if (i >= n) continue;
      const int tl = i / cpr, c = (i % cpr) * 8;
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        const float wk = sw[tl * KT + k];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(wk, v[u][k][q], acc[q]);
      }
      const long o = (t0 + tl) * d + c;
      if (add) {
        float a8[8];
        load8(add + o, a8);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] += a8[q];
      }
      store8(out + o, acc);
    }
  }
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

int perm_nbits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

}  // namespace

// tokens per workgroup of the row scatter and of the combine: about
// `bytes` of token rows, at most kScatterThreads copies. Measured on the
// Mixtral-, DeepSeek-V3- and Qwen-MoE-like layers: 32 KB for the scatter
// (permute stage 5.64 -> 5.72 TB/s, 4.95 -> 5.27, 3.76 -> 3.86), and for
// the combine 64 KB at K <= 2 (32 KB: 5.44 -> 5.35 TB/s) but 32 KB at
// larger K (5.45 -> 5.56, 4.88 -> 5.07)
int scatter_tokens_per_block(int K, long row_bytes, long bytes = 32768) {
  long tpb = bytes / (row_bytes > 0 ? row_bytes : 1);
  if (tpb < 1) tpb = 1;
  if (tpb > kScatterThreads / K) tpb = kScatterThreads / K;
  return (int)tpb;
}

bool scan_in_scatter(int TK, int E) {
  return (long)E * ((TK + kPermChunk - 1) / kPermChunk) <= kScatterThreads;
}

hipError_t launch_hist_rank_scan(const int32_t* idx, int TK, int E,
                                 int32_t* block_hist, int32_t* rank,
                                 int32_t* counts, int32_t* offsets,
                                 int32_t* const* tile_off, hipStream_t s,
                                 bool scan, bool hist) {
  const int nblk = (TK + kPermChunk - 1) / kPermChunk;
  if (hist)
    hipLaunchKernelGGL(hist_rank_kernel, dim3(nblk), dim3(kRankWaves * kWave), 0,
                       s, idx, TK, E, perm_nbits(E), block_hist, rank);
  if (!scan) return hipGetLastError();
  TileOffPtrs tp;
  for (int i = 0; i < kNumTileBM; ++i) tp.p[i] = tile_off[i];
  int ep = 1;
  while (ep < E) ep <<= 1;
  const int tpe = 1024 / ep;  // threads per expert (E <= 1024)
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, block_hist, nblk,
                     E, tpe, counts, offsets, tp);
  return hipGetLastError();
}

hipError_t launch_slots(const int32_t* idx, const int32_t* first,
                        const int32_t* rank, int TK, int E, int32_t* dest,
                        int32_t* sorted_src, hipStream_t s) {
  hipLaunchKernelGGL(slots_kernel, dim3((unsigned)((TK + 255) / 256)), dim3(256),
                     0, s, idx, first, rank, (long)TK, E, dest, sorted_src);
  return hipGetLastError();
}

hipError_t launch_tile_prefix(const int32_t* offsets, int E,
                              int32_t* const* tile_off, hipStream_t s) {
  TileOffPtrs tp;
  for (int i = 0; i < kNumTileBM; ++i) tp.p[i] = tile_off[i];
  hipLaunchKernelGGL(tile_prefix_kernel, dim3(1), dim3(1024), 0, s, offsets, E, tp);
  return hipGetLastError();
}

hipError_t launch_scatter(const void* x, const int32_t* idx,
                          const int32_t* first, const int32_t* rank, int T,
                          int E, int K, long row_bytes, int32_t* dest,
                          int32_t* sorted_src, void* x_perm, hipStream_t s,
                          int32_t* counts, int32_t* offsets,
                          int32_t* const* tile_off) {
  const int tpb = scatter_tokens_per_block(K, row_bytes);
  const long blocks = (T + tpb - 1) / tpb;
  const int TK = T * K;
  TileOffPtrs tp{};
  if (counts)
    for (int i = 0; i < kNumTileBM; ++i) tp.p[i] = tile_off[i];
  if (counts && scan_in_scatter(TK, E))
    hipLaunchKernelGGL(scatter_kernel<true>, dim3((unsigned)blocks),
                       dim3(kScatterThreads), 0, s, (const u32x4*)x, idx, first,
                       rank, T, E, K, (int)(row_bytes / 16), tpb, dest,
                       sorted_src, (u32x4*)x_perm,
                       (TK + kPermChunk - 1) / kPermChunk, counts, offsets, tp);
  else
    hipLaunchKernelGGL(scatter_kernel<false>, dim3((unsigned)blocks),
                       dim3(kScatterThreads), 0, s, (const u32x4*)x, idx, first,
                       rank, T, E, K, (int)(row_bytes / 16), tpb, dest,
                       sorted_src, (u32x4*)x_perm, 0, nullptr, nullptr, tp);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_combine_t(const T* y, const int32_t* dest, const float* w,
                            const T* add, T* out, int Ttok, int K, int d,
                            hipStream_t s) {
  const int tpb = scatter_tokens_per_block(K, (long)d * sizeof(T),
                                           K <= 2 ? 65536 : 32768);
  const dim3 grid((unsigned)((Ttok + tpb - 1) / tpb)), block(kScatterThreads);
  if (K == 2)
    hipLaunchKernelGGL((combine_k_kernel<T, 8, 2>), grid, block, 0, s, y, dest, w,
                       add, out, Ttok, d, tpb);
  else if (K == 4)
    hipLaunchKernelGGL((combine_k_kernel<T, 2, 4>), grid, block, 0, s, y, dest, w,
                       add, out, Ttok, d, tpb);
  else if (K == 8)
    hipLaunchKernelGGL((combine_k_kernel<T, 1, 8>), grid, block, 0, s, y, dest, w,
                       add, out, Ttok, d, tpb);
  else if (K >= 8)
    hipLaunchKernelGGL((combine_kernel<T, 1>), grid, block, 0, s, y, dest, w, add,
                       out, Ttok, K, d, tpb);
  else if (K >= 4)
    hipLaunchKernelGGL((combine_kernel<T, 2>), grid, block, 0, s, y, dest, w, add,
                       out, Ttok, K, d, tpb);
  else
    hipLaunchKernelGGL((combine_kernel<T, 4>), grid, block, 0, s, y, dest, w, add,
                       out, Ttok, K, d, tpb);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* y, const int32_t* dest,
                          const float* w, const void* add, void* out, int T,
                          int K, int d, hipStream_t s) {
  if (dtype == MOE_F32)
    return launch_combine_t((const float*)y, dest, w, (const float*)add,
                            (float*)out, T, K, d, s);
  return launch_combine_t((const bf16*)y, dest, w, (const bf16*)add, (bf16*)out,
                          T, K, d, s);
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
