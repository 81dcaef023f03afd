// Stable ranking of one chunk of token copies by expert (device code shared
// by the permute's histogram kernel and the fused top-K kernel).
#pragma once

#include "launch.h"

namespace moe {

// Copies of chunk b are j = b * kPermChunk + i, i < n (n <= kPermChunk), with
// expert e_at(i). NRW waves each walk kPermChunk / NRW consecutive copies, 64
// at a time: the lanes holding the same expert are found with nbits ballots
// (nbits = ceil(log2 E)) and ranked by popcount against a per-wave count in
// LDS. A prefix over the waves then makes every rank chunk-wide, so copies
// of one expert are ranked in copy order (stable). Writes the chunk's
// histogram hist_row[e] (its count of each expert) and rank[j]. cnt is
// NRW * EM ints of LDS (E <= EM); every thread of the NRW waves calls this.
template <int NRW, int EM, typename EAt>
__device__ __forceinline__ void rank_chunk(EAt e_at, int n, int E, int nbits,
                                           long j0, int32_t (*cnt)[EM],
                                           int32_t* __restrict__ hist_row,
                                           int32_t* __restrict__ rank) {
  constexpr int PER = kPermChunk / NRW, R = PER / kWave;
  static_assert(PER % kWave == 0, "chunk split");
  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  for (int i = tid; i < NRW * E; i += NRW * kWave) cnt[i / E][i % E] = 0;
  __syncthreads();
  int ex[R], rk[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = w * PER + r * kWave + lane;
    const bool valid = i < n;
    const int e = valid ? e_at(i) : 0;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bal = __ballot(valid && on);
      m &= on ? bal : ~bal;
    }
    ex[r] = e;
    rk[r] = 0;
    if (valid) {
      const int base = cnt[w][e];  // every lane of the group reads first
      rk[r] = base + __popcll(m & ((1ull << lane) - 1ull));
    }
    __builtin_amdgcn_wave_barrier();
    if (valid && (m >> lane) == 1ull) cnt[w][e] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // per expert: chunk count, and each wave's first rank (in place)
  for (int e = tid; e < E; e += NRW * kWave) {
    int run = 0;
#pragma unroll
    for (int q = 0; q < NRW; ++q) {
      const int c = cnt[q][e];
      cnt[q][e] = run;
      run += c;
    }
    hist_row[e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = w * PER + r * kWave + lane;
    if (i < n) rank[j0 + i] = cnt[w][ex[r]] + rk[r];
  }
}

}  // namespace moe
