// Shared definitions of the MoE library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Kernel-choice switches read from the environment (MOE_GEMM_BACKEND,
// MOE_BIG_TILE_WAVES, MOE_TILE_GROUP_N, MOE_WGRAD_T) exist only in builds
// compiled with -DMOE_TUNING, which serve to measure alternatives; the
// library otherwise ignores the environment and always makes its own
// choices.
inline const char* tuning_env(const char* name) {
#ifdef MOE_TUNING
  return getenv(name);
#else
  (void)name;
  return nullptr;
#endif
}
constexpr int kNumXcd = 8;  // MI355X: 8 XCDs, workgroups dispatched round-robin

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bf16 with round-to-nearest-even (NaN stays NaN).
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return (bf16)v;
}

// Remap a workgroup id so that each XCD receives one contiguous range of
// logical ids: workgroup b runs on XCD b % 8, so logical id =
// (b % 8) * (n / 8) + b / 8. n must be a multiple of 8.
__host__ __device__ inline int xcd_remap(int b, int n) {
  return (b % kNumXcd) * (n / kNumXcd) + b / kNumXcd;
}

// The same for any n: a bijection of [0, n) that hands each XCD a
// contiguous range of logical indices whose sizes differ by at most one.
__host__ __device__ inline int xcd_remap_n(int b, int n) {
  const int x = b % kNumXcd, q = n / kNumXcd, r = n % kNumXcd;
  return x * q + (x < r ? x : r) + b / kNumXcd;
}

// Largest g in [0, G) with pre[g] <= v (pre is non-decreasing, pre[0] = 0).
__host__ __device__ inline int upper_group(const int32_t* pre, int G, int v) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= v) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Grouped GEMM problem, shared by the MFMA and the SIMT kernels.
//
// Logical product: C[i, j] = sum_k A(i, k) * B(j, k), fp32 accumulation.
//   A(i, k) = A[i * lda + k]            (a_kc: k contiguous)
//           = A[k * lda + i]            (otherwise: i contiguous)
//   B(j, k) = B[g * sB + j * ldb + k]   (b_kc)
//           = B[g * sB + k * ldb + j]   (otherwise)
// Scheduling:
//   kSchedM  rows i are grouped: group g owns rows [off[g], off[g+1]) of A
//            and C and uses B_g; off == nullptr means one group of M rows.
//            tile_off[g] = sum_{g' < g} ceil(count_g' / BM).
//   kSchedK  the contraction index k is grouped: group g sums over
//            k in [off[g], off[g+1]) and writes C_g = C + g * sC, an
//            [M, N] matrix; B has no group stride. An empty group writes 0.
// K-concatenation: for k >= K1 the operands are A2 / B2 (same layouts),
// indexed with k - K1 (K1 a multiple of the k-tile).
// Dual: a second B operand B2 gives a second accumulator (same A).
// ---------------------------------------------------------------------------
enum : int { kSchedM = 0, kSchedK = 1 };
enum : int {
  kEpiStore = 0,      // C = acc
  kEpiSwiglu = 1,     // C = silu(acc) * acc2; C2 = acc, C3 = acc2 if set
  kEpiSwigluBwd = 2,  // dh = acc; C = dh * b * silu'(a), C2 = dh * silu(a)
  kEpiSwigluMx = 3,   // h = silu(acc) * acc2 as MXFP8: C = E4M3 codes [M, N],
                      // C2 = E8M0 scales [M, N/32] (blocks along N)
  kEpiStoreF32 = 4,   // C = acc in fp32 (partial sums)
  kEpiAccum = 5,      // C = C + acc (read, add in fp32, one rounding)
};

struct GemmParams {
  int M, N, K, K1, G;
  const int32_t* off;
  const int32_t* tile_off;
  const void* A; const void* A2; long lda;
  const void* B; const void* B2; long ldb; long sB;
  void* C; void* C2; void* C3; long ldc; long sC;
  const void* aux_a; const void* aux_b;  // kEpiSwigluBwd: saved a, b (ld = ldc)
  int tiles_m_max;                      // upper bound of row tiles (kSchedM)
  int group_n;                          // n-tiles per rasterization group
  // MXFP8 operands: E8M0 scales per 32 elements along k in the
  // span-grouped layout ([K/128][rows][4], mx_scale_index): A's array has
  // s_rows rows (all of A's rows, also when they are gathered); B's stacks
  // the groups' N-row operands (G * N rows when grouped by rows, else N);
  // the quantising epilogue writes C's scales for M rows.
  const uint8_t* As; const uint8_t* Bs; const uint8_t* B2s;
  long s_rows;
  // gathered A rows (direct-to-LDS GEMM 1 only): row i of A (and of As)
  // is row gsrc[i] / gdiv of the A given, e.g. token t of copy j = t*K+k
  const int32_t* gsrc; int gdiv;
  // kEpiSwigluMx: optional bf16 copies of the pre-activations (ld = ldc)
  void* Sa; void* Sb;
  // kSchedK: the group ranges are off[g] * kmul (0 means 1)
  int kmul;
  // kSchedM big tiles: row x column tiles that run at once (one per CU),
  // for the split of a partial last round into quarter tiles; 0 = no
  // split, -1 = the device's CU count (resolved by the launcher)
  int slots;
  // kSchedK: the rows contracted over all groups (the sum of the group
  // ranges), a hint for the kernel choice known on the host; 0 = unknown
  long k_total;
};

}  // namespace moe
