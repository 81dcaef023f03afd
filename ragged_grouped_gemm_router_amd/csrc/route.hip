// Top-K gate: one wavefront per token.
//
// Each lane holds ceil(E/64) candidates as 64-bit keys: the high word is
// the selection key mapped to an unsigned integer whose order is the
// float order (-0.0 folded onto +0.0, NaN onto -inf), the low word is
// ~expert_id, so the unsigned maximum is the largest key and, among equal
// keys, the lowest expert id. K rounds of a lane-local max plus a 6-step
// butterfly max over the wave pick the winners in (key desc, id asc)
// order; the owning lane retires each winner. Lanes 0..K-1 then hold the
// K winners and form the renormalised weights with two wave reductions.
#include "launch.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t b = __float_as_uint(v);
  if (v == 0.0f) b = 0u;                // -0.0 ties +0.0
  if (v != v) b = 0xff800000u;          // NaN counts as -inf
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
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

template <int CPL>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T,
    int E, int K, int gate, int32_t* __restrict__ idx,
    float* __restrict__ wout) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const float* L = logits + (long)t * E;

  uint64_t key[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + kWave * c;
    if (e < E) {
      float v = L[e];
      if (bias) v = v + bias[e];
      key[c] = ((uint64_t)orderable(v) << 32) | (uint32_t)(~(uint32_t)e);
    } else {
      key[c] = 0;  // below every real key (-inf maps to 0x007fffff)
    }
  }

  int mine = -1;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int c = 0; c < CPL; ++c) best = key[c] > best ? key[c] : best;
    best = wave_max_u64(best);
    const int e = (int)(~(uint32_t)best);
    if ((e & (kWave - 1)) == lane) {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        if (c == (e >> 6)) key[c] = 0;
    }
    if (lane == k) mine = e;
  }

  // weights from the raw logits of the winners (lanes 0..K-1)
  const bool act = lane < K;
  const float l = act ? L[mine] : 0.0f;
  float z;
  if (gate == MOE_GATE_SOFTMAX) {
    const float mx = wave_max(act ? l : -INFINITY);
    z = act ? expf(l - mx) : 0.0f;
  } else {
    z = act ? 1.0f / (1.0f + expf(-l)) : 0.0f;
  }
  const float s = wave_sum(z);
  if (act) {
    idx[(long)t * K + lane] = mine;
    wout[(long)t * K + lane] = s > 0.0f ? z / s : 1.0f / (float)K;
  }
}

}  // namespace

hipError_t launch_topk(const float* logits, const float* bias, int T, int E,
                       int K, int gate, int32_t* idx, float* w,
                       hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  const int cpl = (E + kWave - 1) / kWave;
  if (cpl <= 1)
    hipLaunchKernelGGL(topk_kernel<1>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w);
  else if (cpl <= 2)
    hipLaunchKernelGGL(topk_kernel<2>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w);
  else if (cpl <= 4)
    hipLaunchKernelGGL(topk_kernel<4>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w);
  else if (cpl <= 8)
    hipLaunchKernelGGL(topk_kernel<8>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w);
  else
    hipLaunchKernelGGL(topk_kernel<16>, grid, block, 0, s, logits, bias, T, E, K, gate, idx, w);
  return hipGetLastError();
}

}  // namespace moe

namespace moe {
namespace {

// Gate backward, one wavefront per token: d loss / d logits from
// d loss / d topk_w. Lane e writes logit e (and e + 64, ...) once: the
// selected ones get w_k (d_w_k - <w, d_w>) (softmax) or
// s_k (1 - s_k) / S (d_w_k - <w, d_w>) with s = sigmoid(logit), S the sum
// of the selected s (sigmoid; zero if S == 0, where the weights were 1/K);
// the rest get zero. Also the same values in the activation dtype.
template <typename TA>
__global__ __launch_bounds__(256) void router_grad_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const float* __restrict__ d_w, int T, int E,
    int K, int gate, float* __restrict__ d_logits, TA* __restrict__ d_logits_a) {
  const int lane = threadIdx.x % kWave;
  const int t = blockIdx.x * (256 / kWave) + threadIdx.x / kWave;
  if (t >= T) return;
  const long r = (long)t * K;
  float inner = 0.0f, S = 0.0f;
  for (int k = 0; k < K; ++k) {
    inner = fmaf(w[r + k], d_w[r + k], inner);
    if (gate == MOE_GATE_SIGMOID) {
      const float l = logits[(long)t * E + idx[r + k]];
      S += 1.0f / (1.0f + expf(-l));
    }
  }
  for (int e = lane; e < E; e += kWave) {
    float g = 0.0f;
    for (int k = 0; k < K; ++k) {
      if (idx[r + k] != e) continue;
      const float dd = d_w[r + k] - inner;
      if (gate == MOE_GATE_SOFTMAX) {
        g = w[r + k] * dd;
      } else if (S > 0.0f) {
        const float s = 1.0f / (1.0f + expf(-logits[(long)t * E + e]));
        g = s * (1.0f - s) / S * dd;
      }
    }
    d_logits[(long)t * E + e] = g;
    d_logits_a[(long)t * E + e] = (TA)g;
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
                              const float* d_w, int T, int E, int K, int gate,
                              float* d_logits, void* d_logits_a, int G,
                              int32_t* split, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(router_grad_kernel<float>, grid, block, 0, s, logits,
                       idx, w, d_w, T, E, K, gate, d_logits, (float*)d_logits_a);
  else
    hipLaunchKernelGGL(router_grad_kernel<bf16>, grid, block, 0, s, logits, idx,
                       w, d_w, T, E, K, gate, d_logits, (bf16*)d_logits_a);
  hipLaunchKernelGGL(split_kernel, dim3(1), dim3(1024), 0, s, T, G, split);
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
