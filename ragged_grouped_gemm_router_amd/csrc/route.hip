// Top-K gate: one wavefront per token.
//
// Each lane holds ceil(E/64) candidates (expert e = lane + 64 c) with a
// 32-bit selection key: the selection value mapped to an unsigned integer
// whose order is the float order (-0.0 folded onto +0.0, NaN onto -inf).
// The K-th largest key is found by a 32-step binary search on its bits,
// each step counting the candidates at or above a trial value with one
// ballot per candidate slot. The winners are the keys above it and, among
// the keys equal to it, the lowest expert ids. They are compacted in id
// order into LDS; lanes 0..K-1 then take one winner each, rank it (key
// descending, id ascending: the output order) and form the renormalised
// weight from the winners' raw logits.
//
// Split router GEMM (G > 1): `logits` holds G partial products of the
// logits, pstride floats apart; both kernels sum a token's partials in the
// order g = 0, 1, .., G - 1 (fp32), write that sum to lout and select
// from it.
#include "launch.h"
#include "rank.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t b = __float_as_uint(v);
  if (v == 0.0f) b = 0u;                // -0.0 ties +0.0
  if (v != v) b = 0xff800000u;          // NaN counts as -inf
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// number of lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <int CPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int K, int gate, int32_t* __restrict__ idx,
    float* __restrict__ wout, int G, long pstride, float* __restrict__ lout) {
  __shared__ uint32_t s_key[4][MOE_K_MAX];
  __shared__ int32_t s_id[4][MOE_K_MAX];
  __shared__ float s_l[4][MOE_K_MAX];
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  const int t = blockIdx.x * (256 / kWave) + wv;
  if (t >= T) return;  // (the whole wave)
  const float* L = logits + (long)t * E;

  float lg[CPL];
  uint32_t key[CPL];  // 0 marks padding: every real key is above it
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + kWave * c;
    lg[c] = 0.0f;
    key[c] = 0u;
    if (e < E) {
      // every partial's load issued at once (clamped to the last one),
      // added in order while g < G
      float v = L[e];
      if (G > 1) {
        float pv[kRouterMaxSplit];
#pragma unroll
        for (int g = 1; g < kRouterMaxSplit; ++g) pv[g] = L[min(g, G - 1) * pstride + e];
#pragma unroll
        for (int g = 1; g < kRouterMaxSplit; ++g) v = g < G ? v + pv[g] : v;
        lout[(long)t * E + e] = v;
      }
      lg[c] = v;
      key[c] = orderable(bias ? v + bias[e] : v);
    }
  }
  // the K-th largest key: the largest value with at least K keys at or
  // above it (E >= K real keys, all >= 0x007fffff, so it is one of them)
  uint32_t thr = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial = thr | (1u << bit);
    int n = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) n += __popcll(__ballot(key[c] >= trial));
    if (n >= K) thr = trial;
  }
  // winners: every key above thr, then the lowest ids among keys equal to
  // it (ids ascend with c, then with the lane)
  int need = K;
#pragma unroll
  for (int c = 0; c < CPL; ++c) need -= __popcll(__ballot(key[c] > thr));
  int base = 0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const uint64_t eq = __ballot(key[c] == thr);
    const bool win = key[c] > thr || (key[c] == thr && lanes_below(eq) < need);
    need -= __popcll(eq);
    const uint64_t wm = __ballot(win);
    if (win) {
      const int p = base + lanes_below(wm);
      s_key[wv][p] = key[c];
      s_id[wv][p] = lane + kWave * c;
      s_l[wv][p] = lg[c];
    }
    base += __popcll(wm);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (lane >= K) return;
  // rank of this lane's winner, and the weights over the K raw logits
  const uint32_t mk = s_key[wv][lane];
  const float l = s_l[wv][lane];
  int rank = 0;
  float mx = -INFINITY;
  for (int j = 0; j < K; ++j) {
    const uint32_t kj = s_key[wv][j];
    rank += kj > mk || (kj == mk && j < lane);
    mx = fmaxf(mx, s_l[wv][j]);
  }
  float sum = 0.0f;
  for (int j = 0; j < K; ++j) {
    const float lj = s_l[wv][j];
    sum += gate == MOE_GATE_SOFTMAX ? expf(lj - mx) : 1.0f / (1.0f + expf(-lj));
  }
  const float z = gate == MOE_GATE_SOFTMAX ? expf(l - mx) : 1.0f / (1.0f + expf(-l));
  idx[(long)t * K + rank] = s_id[wv][lane];
  wout[(long)t * K + rank] = sum > 0.0f ? z / sum : 1.0f / (float)K;
}

// Top-K with the permute's chunk ranking fused in, for E <= 32 with E a
// multiple of 4, and K a divisor of kPermChunk: workgroup b takes the
// kPermChunk / K tokens whose copies form permute chunk b, one thread per
// token. A thread loads its token's row of logits in 16-byte pieces (EP/4
// loads issued together; EP >= E, a multiple of 4), selects its K experts
// by K passes over the E candidates (largest orderable key, lowest id
// among equal keys: the same order as the wave kernel), then forms the
// renormalised weights from the raw logits of the winners. The workgroup
// then ranks the chunk's copies by expert (rank_chunk), so the permute
// needs no histogram pass of its own.
template <int NW, int EP>
__global__ __launch_bounds__(NW * kWave) void topk_rank_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int K, int gate, int nbits, int32_t* __restrict__ idx,
    float* __restrict__ wout, int32_t* __restrict__ block_hist,
    int32_t* __restrict__ rank, int G, long pstride, float* __restrict__ lout) {
  constexpr int CT = NW * kWave;  // tokens of the chunk (= kPermChunk / K)
  constexpr int KC = kPermChunk / CT;  // = K
  constexpr int NQ = EP / 4;
  __shared__ int32_t sidx[kPermChunk];
  __shared__ int32_t cnt[NW][32];
  const int tl = threadIdx.x;
  const long t = (long)blockIdx.x * CT + tl;
  if (t < T) {
    const float* L = logits + t * E;
    f32x4 v[NQ], bv[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {  // clamped addresses: no branch between
      const int c = min(4 * q, E - 4);
      v[q] = *(const f32x4*)(L + c);
      bv[q] = bias ? *(const f32x4*)(bias + c) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (G > 1) {  // (as the wave kernel: all loads first, then in order)
      f32x4 pv[kRouterMaxSplit - 1][NQ];
#pragma unroll
      for (int g = 1; g < kRouterMaxSplit; ++g)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
          pv[g - 1][q] = *(const f32x4*)(L + min(g, G - 1) * pstride + min(4 * q, E - 4));
#pragma unroll
      for (int g = 1; g < kRouterMaxSplit; ++g)
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) v[q][i] = g < G ? v[q][i] + pv[g - 1][q][i] : v[q][i];
    }
    if (G > 1) {
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (4 * q < E) *(f32x4*)(lout + t * E + 4 * q) = v[q];
    }
    uint32_t key[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) {
      const float x = v[e / 4][e % 4];
      // the key is fp32(logit + bias) with a bias, the logit without one
      key[e] = e < E ? orderable(bias ? x + bv[e / 4][e % 4] : x) : 0u;
    }
    int sel[KC];  // K winners, in (key desc, id asc) order
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      // every real key is above 0 (-inf maps to 0x007fffff), so 0 marks
      // padding and retired candidates; the first largest key wins
      uint32_t bk = 0;
      int be = 0;
#pragma unroll
      for (int e = 0; e < EP; ++e) {
        const bool better = key[e] > bk;
        bk = better ? key[e] : bk;
        be = better ? e : be;
      }
      sel[k] = be;
#pragma unroll
      for (int e = 0; e < EP; ++e) key[e] = e == be ? 0u : key[e];
    }
    float l[KC], z[KC];
    float mx = -INFINITY, sum = 0.0f;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      float x = 0.0f;
#pragma unroll
      for (int e = 0; e < EP; ++e) x = e == sel[k] ? v[e / 4][e % 4] : x;
      l[k] = x;
      mx = fmaxf(mx, x);
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      z[k] = gate == MOE_GATE_SOFTMAX ? expf(l[k] - mx) : 1.0f / (1.0f + expf(-l[k]));
      sum += z[k];
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      idx[t * KC + k] = sel[k];
      wout[t * KC + k] = sum > 0.0f ? z[k] / sum : 1.0f / (float)KC;
      sidx[tl * KC + k] = sel[k];
    }
  }
  __syncthreads();
  const long j0 = (long)blockIdx.x * kPermChunk;
  const int n = (int)min((long)kPermChunk, (long)T * K - j0);
  rank_chunk<NW, 32>([&](int i) { return sidx[i]; }, n, E, nbits, j0, cnt,
                     block_hist + (long)blockIdx.x * E, rank);
}

template <int NW>
hipError_t launch_topk_rank_nw(const float* logits, const float* bias, int T,
                               int E, int K, int gate, int nbits, int32_t* idx,
                               float* w, int32_t* block_hist, int32_t* rank,
                               int G, float* lout, hipStream_t s) {
  const dim3 grid((unsigned)((T + NW * kWave - 1) / (NW * kWave))), block(NW * kWave);
  const long ps = (long)T * E;
  if (E <= 8)
    hipLaunchKernelGGL((topk_rank_kernel<NW, 8>), grid, block, 0, s, logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, ps, lout);
  else if (E <= 16)
    hipLaunchKernelGGL((topk_rank_kernel<NW, 16>), grid, block, 0, s, logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, ps, lout);
  else
    hipLaunchKernelGGL((topk_rank_kernel<NW, 32>), grid, block, 0, s, logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, ps, lout);
  return hipGetLastError();
}

}  // namespace

// (up to 32 experts: with more, one thread's serial selection costs more
// than the histogram pass it saves; measured on the 60-expert layer)
bool topk_rank_supported(int E, int K) {
  return E >= 4 && E <= 32 && E % 4 == 0 && K >= 1 && kPermChunk % K == 0 &&
         kPermChunk / K >= kWave;
}

hipError_t launch_topk_rank(const float* logits, const float* bias, int T,
                            int E, int K, int gate, int32_t* idx, float* w,
                            int32_t* block_hist, int32_t* rank, hipStream_t s,
                            int G, float* lout) {
  if (G < 1 || G > kRouterMaxSplit || (G > 1 && !lout)) return hipErrorInvalidValue;
  if (!topk_rank_supported(E, K)) return hipErrorNotSupported;
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  switch (kPermChunk / K / kWave) {  // waves per workgroup: 16 / K
    case 16: return launch_topk_rank_nw<16>(logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, lout, s);
    case 8: return launch_topk_rank_nw<8>(logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, lout, s);
    case 4: return launch_topk_rank_nw<4>(logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, lout, s);
    case 2: return launch_topk_rank_nw<2>(logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, lout, s);
    default: return launch_topk_rank_nw<1>(logits, bias, T, E, K, gate, nbits, idx, w, block_hist, rank, G, lout, s);
  }
}

hipError_t launch_topk(const float* logits, const float* bias, int T, int E,
                       int K, int gate, int32_t* idx, float* w, hipStream_t s,
                       int G, float* lout) {
  if (G < 1 || G > kRouterMaxSplit || (G > 1 && !lout)) return hipErrorInvalidValue;
  const dim3 grid((T + 3) / 4), block(256);
  const int cpl = (E + kWave - 1) / kWave;
  const long ps = (long)T * E;
  if (cpl <= 1)
    hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w, G, ps, lout);
  else if (cpl <= 2)
    hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w, G, ps, lout);
  else if (cpl <= 4)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w, G, ps, lout);
  else if (cpl <= 8)
    hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w, G, ps, lout);
  else
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w, G, ps, lout);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
namespace {

__device__ __forceinline__ float sigmoidf(float l) {
  return 1.0f / (1.0f + expf(-l));
}

// The gate's probability of every expert for one token, as the balance
// statistics define it: softmax over all E logits (softmax gate) or the
// sigmoids over their sum (sigmoid gate; 1/E each if every sigmoid is
// zero). Each lane visits experts lane, lane + 64, ...; the wave-wide
// max and sum leave the same value in every lane. Returns the
// normaliser; the probability of expert e is then prob(row[e]).
struct GateProbs {
  int gate;
  float m, z;
  __device__ GateProbs(const float* row, int E, int gate_, int lane)
      : gate(gate_), m(0.0f), z(0.0f) {
    if (gate == MOE_GATE_SOFTMAX) {
      float mx = -INFINITY;
      for (int e = lane; e < E; e += kWave) mx = fmaxf(mx, row[e]);
      m = wave_max(mx);
      float zz = 0.0f;
      for (int e = lane; e < E; e += kWave) zz += expf(row[e] - m);
      z = wave_sum(zz);
    } else {
      float zz = 0.0f;
      for (int e = lane; e < E; e += kWave) zz += sigmoidf(row[e]);
      z = wave_sum(zz);
    }
  }
  __device__ float num(float l) const {
    return gate == MOE_GATE_SOFTMAX ? expf(l - m) : sigmoidf(l);
  }
  __device__ float prob(float l, int E) const {
    return z > 0.0f ? num(l) / z : 1.0f / (float)E;
  }
};

// Gate backward, one wavefront per token: d loss / d logits from
// d loss / d topk_w. Lane e writes logit e (and e + 64, ...) once: the
// selected ones get w_k (d_w_k - <w, d_w>) (softmax) or
// s_k (1 - s_k) / S (d_w_k - <w, d_w>) with s = sigmoid(logit), S the sum
// of the selected s (sigmoid; zero if S == 0, where the weights were 1/K);
// the rest get zero. With counts given, every logit j also gets
// aux_coef (E / T) q_j (f_j - sum_i f_i P_i), the gradient of the balance
// loss E sum_i f_i mean_t P_ti at fixed f = counts / T, where P is the
// full-row gate probability and q_j = P_j (softmax) or
// s_j (1 - s_j) / sum_i s_i (sigmoid). Also the same values in the
// activation dtype, in rows of ld_a >= E elements whose tail is zero.
template <typename TA>
__global__ __launch_bounds__(256) void router_grad_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const float* __restrict__ d_w,
    const int32_t* __restrict__ counts, float aux_coef, int T, int E, int K,
    int gate, float* __restrict__ d_logits, TA* __restrict__ d_logits_a,
    int ld_a) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const long r = (long)t * K;
  const float* row = logits + (long)t * E;
  float inner = 0.0f, S = 0.0f;
  for (int k = 0; k < K; ++k) {
    inner = fmaf(w[r + k], d_w[r + k], inner);
    if (gate == MOE_GATE_SIGMOID) S += sigmoidf(row[idx[r + k]]);
  }
  const bool aux = counts != nullptr;
  const float invT = 1.0f / (float)T;
  float aux_scale = 0.0f, aux_inner = 0.0f;
  GateProbs gp(row, aux ? E : 0, gate, lane);
  if (aux) {
    aux_scale = aux_coef * (float)E * invT;
    float in = 0.0f;
    for (int e = lane; e < E; e += kWave)
      in += ((float)counts[e] * invT) * gp.prob(row[e], E);
    aux_inner = wave_sum(in);
  }
  for (int e = lane; e < E; e += kWave) {
    float g = 0.0f;
    for (int k = 0; k < K; ++k) {
      if (idx[r + k] != e) continue;
      const float dd = d_w[r + k] - inner;
      if (gate == MOE_GATE_SOFTMAX) {
        g = w[r + k] * dd;
      } else if (S > 0.0f) {
        const float s = sigmoidf(row[e]);
        g = s * (1.0f - s) / S * dd;
      }
    }
    if (aux && gp.z > 0.0f) {
      float q;
      if (gate == MOE_GATE_SOFTMAX) {
        q = gp.prob(row[e], E);
      } else {
        const float s = sigmoidf(row[e]);
        q = s * (1.0f - s) / gp.z;
      }
      g += aux_scale * q * ((float)counts[e] * invT - aux_inner);
    }
    d_logits[(long)t * E + e] = g;
    d_logits_a[(long)t * ld_a + e] = (TA)g;
  }
  for (int e = E + lane; e < ld_a; e += kWave)
    d_logits_a[(long)t * ld_a + e] = (TA)0.0f;
}

// Balance statistics, pass 1: block g adds up the gate probabilities of
// tokens [g T / G, (g + 1) T / G) per expert into part[g E + e]. Wave v
// takes every fourth token of the range in order, each lane keeping the
// running sums of its experts; the four waves' sums are then added in
// wave order, so the result does not depend on scheduling.
template <int CPL>
__global__ __launch_bounds__(256) void balance_part_kernel(
    const float* __restrict__ logits, int T, int E, int G, int gate,
    float* __restrict__ part) {
  __shared__ float wsum[4][MOE_E_MAX];
  const int lane = threadIdx.x % kWave, v = threadIdx.x / kWave;
  const int g = blockIdx.x;
  const long t0 = (long)g * T / G, t1 = (long)(g + 1) * T / G;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
  for (long t = t0 + v; t < t1; t += 4) {
    const float* row = logits + t * E;
    const GateProbs gp(row, E, gate, lane);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + kWave * c;
      if (e < E) acc[c] += gp.prob(row[e], E);
    }
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + kWave * c;
    if (e < E) wsum[v][e] = acc[c];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    part[(long)g * E + e] = ((wsum[0][e] + wsum[1][e]) + wsum[2][e]) + wsum[3][e];
}

// Balance statistics, pass 2 (one block of 1024 threads): thread
// (slice q, expert e) adds part[g E + e] for g = q, q + Q, ... with Q =
// 1024 / Ep slices (Ep = E rounded up to a power of two); the Q slice sums
// are then added in slice order. p_mean[e] = that sum / T,
// f[e] = counts[e] / T and aux = E sum_e f[e] p_mean[e], the products
// summed by a fixed tree, so the result does not depend on scheduling.
__global__ __launch_bounds__(1024) void balance_finish_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ counts, int T,
    int E, int Ep, int G, float* __restrict__ f, float* __restrict__ p_mean,
    float* __restrict__ aux) {
  __shared__ float red[1024];
  const int tid = threadIdx.x, Q = 1024 / Ep;
  {
    const int e = tid % Ep, q = tid / Ep;
    float s = 0.0f;
    if (e < E)
      for (int g = q; g < G; g += Q) s += part[(long)g * E + e];
    red[tid] = s;
  }
  __syncthreads();
  float prod = 0.0f;
  if (tid < E) {
    float s = 0.0f;
    for (int q = 0; q < Q; ++q) s += red[q * Ep + tid];
    const float P = s / (float)T, fe = (float)counts[tid] / (float)T;
    p_mean[tid] = P;
    f[tid] = fe;
    prod = fe * P;
  }
  __syncthreads();
  red[tid] = prod;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  if (tid == 0) aux[0] = (float)E * red[0];
}

// Route-bias balance step (one block of 1024 threads): load = counts /
// sum(counts), the sum taken over 64-bit integers; each expert's bias
// moves against the sign of load - target by gamma (rule 0), or by gamma
// times the load clamped below at 1e-6 (rule 1). No contraction, so every
// product and difference rounds once, as written.
__global__ __launch_bounds__(1024) void bias_update_kernel(
    const int32_t* __restrict__ counts, int E, float gamma, float target,
    int rule, float* __restrict__ bias, float* __restrict__ load_out) {
#pragma clang fp contract(off)
  __shared__ long long red[1024];
  const int e = threadIdx.x;
  red[e] = e < E ? counts[e] : 0;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (e < off) red[e] += red[e + off];
    __syncthreads();
  }
  if (e >= E) return;
  const float load = (float)counts[e] / (float)red[0];
  const float tgt = target > 0.0f ? target : 1.0f / (float)E;
  const float sg = load > tgt ? 1.0f : (load < tgt ? -1.0f : 0.0f);
  float step = gamma * sg;
  if (rule == 1) step = step * fmaxf(load, 1e-6f);
  bias[e] = bias[e] - step;
  if (load_out) load_out[e] = load;
}

// Load monitor (one block of 1024 threads): r = mean of the W load rows
// (summed in row order), then min r, the entropy -sum r log(r + 1e-9)
// (fixed tree) and the number of experts with r < 0.3 / E.
__global__ __launch_bounds__(1024) void balance_monitor_kernel(
    const float* __restrict__ hist, int W, int E, float* __restrict__ out) {
#pragma clang fp contract(off)
  __shared__ float rmin[1024], ent[1024];
  __shared__ int cold[1024];
  const int e = threadIdx.x;
  float r = 0.0f;
  if (e < E) {
    float s = 0.0f;
    for (int w = 0; w < W; ++w) s = s + hist[(long)w * E + e];
    r = s / (float)W;
  }
  rmin[e] = e < E ? r : INFINITY;
  ent[e] = e < E ? -(r * logf(r + 1e-9f)) : 0.0f;
  cold[e] = e < E && r < 0.3f / (float)E ? 1 : 0;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (e < off) {
      rmin[e] = fminf(rmin[e], rmin[e + off]);
      ent[e] += ent[e + off];
      cold[e] += cold[e + off];
    }
    __syncthreads();
  }
  if (e == 0) {
    out[0] = rmin[0];
    out[1] = ent[0];
    out[2] = (float)cold[0];
  }
}

// out[i] = sum_g part[g * n + i] in g order (fixed, so deterministic)
template <typename TO>
__global__ __launch_bounds__(256) void reduce_parts_kernel(
    const float* __restrict__ part, long n, int G, TO* __restrict__ out) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int g = 0; g < G; ++g) s += part[g * n + i];
  out[i] = (TO)s;
}

// y[i] += x[i], 8 elements per thread (n % 8 == 0)
template <typename T>
__global__ __launch_bounds__(256) void add_inplace_kernel(
    T* __restrict__ y, const T* __restrict__ x, long n8) {
  const long i = blockIdx.x * 256L + threadIdx.x;
  if (i >= n8) return;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    y[i * 8 + q] = (T)((float)y[i * 8 + q] + (float)x[i * 8 + q]);
}

// split[g] = g * T / G: token ranges of the router-weight partial sums
__global__ void split_kernel(int T, int G, int32_t* __restrict__ split) {
  const int g = threadIdx.x;
  if (g <= G) split[g] = (int)((long)g * T / G);
}

}  // namespace

hipError_t launch_router_grad(int dtype, const float* logits,
                              const int32_t* idx, const float* w,
                              const float* d_w, const int32_t* counts,
                              float aux_coef, int T, int E, int K, int gate,
                              float* d_logits, void* d_logits_a, int ld_a,
                              int G, int32_t* split, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(router_grad_kernel<float>, grid, block, 0, s, logits,
                       idx, w, d_w, counts, aux_coef, T, E, K, gate, d_logits,
                       (float*)d_logits_a, ld_a);
  else
    hipLaunchKernelGGL(router_grad_kernel<bf16>, grid, block, 0, s, logits, idx,
                       w, d_w, counts, aux_coef, T, E, K, gate, d_logits,
                       (bf16*)d_logits_a, ld_a);
  hipLaunchKernelGGL(split_kernel, dim3(1), dim3(1024), 0, s, T, G, split);
  return hipGetLastError();
}

hipError_t launch_balance_stats(const float* logits, const int32_t* counts,
                                int T, int E, int gate, int G, float* part,
                                float* f, float* p_mean, float* aux,
                                hipStream_t s) {
  const int cpl = (E + kWave - 1) / kWave;
  const dim3 grid(G), block(256);
  if (cpl <= 1)
    hipLaunchKernelGGL(balance_part_kernel<1>, grid, block, 0, s, logits, T, E, G, gate, part);
  else if (cpl <= 2)
    hipLaunchKernelGGL(balance_part_kernel<2>, grid, block, 0, s, logits, T, E, G, gate, part);
  else if (cpl <= 4)
    hipLaunchKernelGGL(balance_part_kernel<4>, grid, block, 0, s, logits, T, E, G, gate, part);
  else if (cpl <= 8)
    hipLaunchKernelGGL(balance_part_kernel<8>, grid, block, 0, s, logits, T, E, G, gate, part);
  else
    hipLaunchKernelGGL(balance_part_kernel<16>, grid, block, 0, s, logits, T, E, G, gate, part);
  int Ep = 1;
  while (Ep < E) Ep *= 2;
  hipLaunchKernelGGL(balance_finish_kernel, dim3(1), dim3(1024), 0, s, part,
                     counts, T, E, Ep, G, f, p_mean, aux);
  return hipGetLastError();
}

hipError_t launch_bias_update(const int32_t* counts, int E, float gamma,
                              float target, int rule, float* bias,
                              float* load, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(1024), 0, s, counts, E,
                     gamma, target, rule, bias, load);
  return hipGetLastError();
}

hipError_t launch_balance_monitor(const float* hist, int W, int E, float* out,
                                  hipStream_t s) {
  hipLaunchKernelGGL(balance_monitor_kernel, dim3(1), dim3(1024), 0, s, hist,
                     W, E, out);
  return hipGetLastError();
}

hipError_t launch_split(int T, int G, int32_t* split, hipStream_t s) {
  hipLaunchKernelGGL(split_kernel, dim3(1), dim3(1024), 0, s, T, G, split);
  return hipGetLastError();
}

hipError_t launch_reduce_parts(int dtype, const float* part, long n, int G,
                               void* out, hipStream_t s) {
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(reduce_parts_kernel<float>, grid, block, 0, s, part, n, G,
                       (float*)out);
  else
    hipLaunchKernelGGL(reduce_parts_kernel<bf16>, grid, block, 0, s, part, n, G,
                       (bf16*)out);
  return hipGetLastError();
}

hipError_t launch_add_inplace(int dtype, void* y, const void* x, long n,
                              hipStream_t s) {
  const long n8 = n / 8;
  const dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(add_inplace_kernel<float>, grid, block, 0, s, (float*)y,
                       (const float*)x, n8);
  else
    hipLaunchKernelGGL(add_inplace_kernel<bf16>, grid, block, 0, s, (bf16*)y,
                       (const bf16*)x, n8);
  return hipGetLastError();
}

}  // namespace moe
