// Plain SIMT grouped GEMM: 64x64 output tile per 256-thread workgroup,
// 4x4 outputs per thread, fp32 FMA accumulation, operands staged through
// LDS in k-major order. Serves the fp32 layer and any shape the MFMA
// tiles do not cover. Same problem definition as the MFMA kernels.
#include "gemm.h"

namespace moe {
namespace {

constexpr int BM = kSimtBM, BN = 64, BK = 16, NT = 256;

template <typename T>
__device__ __forceinline__ float ld_a(const GemmParams& p, bool a_kc, int i,
                                      int k) {
  const T* A = (const T*)p.A;
  if (k >= p.K1) { A = (const T*)p.A2; k -= p.K1; }
  return to_f32(a_kc ? A[(long)i * p.lda + k] : A[(long)k * p.lda + i]);
}

template <typename T>
__device__ __forceinline__ float ld_b(const GemmParams& p, const void* Bv,
                                      bool b_kc, int g, int j, int k) {
  const T* B = (const T*)Bv;
  if (k >= p.K1) { B = (const T*)p.B2; k -= p.K1; }
  B += (long)g * p.sB;
  return to_f32(b_kc ? B[(long)j * p.ldb + k] : B[(long)k * p.ldb + j]);
}

__device__ __forceinline__ float sigmoid_acc(float a) {
  return 1.0f / (1.0f + expf(-a));
}

template <typename T, typename TO, bool A_KC, bool B_KC, bool DUAL, int EPI,
          int SCHED>
__global__ __launch_bounds__(NT) void simt_gemm(GemmParams p) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ float B2s[DUAL ? BK : 1][BN + 4];

  const int tid = threadIdx.x;
  const int tiles_n = (p.N + BN - 1) / BN;
  int g = 0, m0, m_end, k_beg = 0, k_end = p.K, nt;
  if (SCHED == kSchedM) {
    int mt = blockIdx.x / tiles_n;
    nt = blockIdx.x % tiles_n;
    if (p.off == nullptr) {
      m0 = mt * BM;
      m_end = p.M;
      if (m0 >= m_end) return;
    } else {
      if (mt >= p.tile_off[p.G]) return;
      g = upper_group(p.tile_off, p.G, mt);
      m0 = p.off[g] + (mt - p.tile_off[g]) * BM;
      m_end = p.off[g + 1];
    }
  } else {
    const int tiles_m = (p.M + BM - 1) / BM;
    g = blockIdx.x / (tiles_m * tiles_n);
    int r = blockIdx.x % (tiles_m * tiles_n);
    m0 = (r / tiles_n) * BM;
    nt = r % tiles_n;
    m_end = p.M;
    k_beg = p.off[g];
    k_end = p.off[g + 1];
  }
  const int n0 = nt * BN;
  const int tx = tid % 16, ty = tid / 16;

  float acc[4][4] = {}, acc2[DUAL ? 4 : 1][DUAL ? 4 : 1] = {};
  for (int k0 = k_beg; k0 < k_end; k0 += BK) {
    for (int e = tid; e < BM * BK; e += NT) {
      // k fastest for k-contiguous operands, rows fastest otherwise
      int i = A_KC ? e / BK : e % BM;
      int kk = A_KC ? e % BK : e / BM;
      int gi = m0 + i, gk = k0 + kk;
      As[kk][i] = (gi < m_end && gk < k_end) ? ld_a<T>(p, A_KC, gi, gk) : 0.f;
    }
    for (int e = tid; e < BN * BK; e += NT) {
      int j = B_KC ? e / BK : e % BN;
      int kk = B_KC ? e % BK : e / BN;
      int gj = n0 + j, gk = k0 + kk;
      bool ok = gj < p.N && gk < k_end;
      Bs[kk][j] = ok ? ld_b<T>(p, p.B, B_KC, SCHED == kSchedM ? g : 0, gj, gk)
                     : 0.f;
      if (DUAL)
        B2s[kk][j] = ok ? ld_b<T>(p, p.B2, B_KC, g, gj, gk) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = As[kk][ty * 4 + r];
#pragma unroll
      for (int c = 0; c < 4; ++c) b[c] = Bs[kk][tx * 4 + c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
      if (DUAL) {
#pragma unroll
        for (int c = 0; c < 4; ++c) b[c] = B2s[kk][tx * 4 + c];
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc2[DUAL ? r : 0][DUAL ? c : 0] =
                fmaf(a[r], b[c], acc2[DUAL ? r : 0][DUAL ? c : 0]);
      }
    }
    __syncthreads();
  }

  TO* C = (TO*)p.C + (SCHED == kSchedK ? (long)g * p.sC : 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = m0 + ty * 4 + r;
    if (i >= m_end) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = n0 + tx * 4 + c;
      if (j >= p.N) continue;
      const long o = (long)i * p.ldc + j;
      if (EPI == kEpiStore) {
        C[o] = from_f32<TO>(acc[r][c]);
      } else if (EPI == kEpiSwiglu) {
        float a = acc[r][c], b = acc2[DUAL ? r : 0][DUAL ? c : 0];
        if (C) C[o] = from_f32<TO>(a * sigmoid_acc(a) * b);
        if (p.C2) ((TO*)p.C2)[o] = from_f32<TO>(a);
        if (p.C3) ((TO*)p.C3)[o] = from_f32<TO>(b);
      } else {  // kEpiSwigluBwd
        float dh = acc[r][c];
        float a = to_f32(((const T*)p.aux_a)[o]);
        float b = to_f32(((const T*)p.aux_b)[o]);
        float s = sigmoid_acc(a);
        C[o] = from_f32<TO>(dh * b * s * (1.0f + a * (1.0f - s)));
        ((TO*)p.C2)[o] = from_f32<TO>(dh * a * s);
      }
    }
  }
}

template <typename T, typename TO, bool A_KC, bool B_KC, bool DUAL, int EPI,
          int SCHED>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  const long tiles_n = (p.N + BN - 1) / BN;
  long tiles = SCHED == kSchedM ? (long)p.tiles_m_max * tiles_n
                                : (long)p.G * ((p.M + BM - 1) / BM) * tiles_n;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((simt_gemm<T, TO, A_KC, B_KC, DUAL, EPI, SCHED>),
                     dim3((unsigned)tiles), dim3(NT), 0, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(GemmOp op, const GemmParams& p, hipStream_t s) {
  switch (op) {
    case kOpRouter:
      return launch<T, float, true, true, false, kEpiStore, kSchedM>(p, s);
    case kOpGemm1:
      return launch<T, T, true, true, true, kEpiSwiglu, kSchedM>(p, s);
    case kOpGemm2:
      return launch<T, T, true, true, false, kEpiStore, kSchedM>(p, s);
    case kOpDgrad2:
      return launch<T, T, true, false, false, kEpiSwigluBwd, kSchedM>(p, s);
    case kOpDgrad1:
      return launch<T, T, true, false, false, kEpiStore, kSchedM>(p, s);
    case kOpWgrad:
      return launch<T, T, false, false, false, kEpiStore, kSchedK>(p, s);
    case kOpRouterDx:
      return launch<T, T, true, false, false, kEpiStore, kSchedM>(p, s);
    case kOpRouterDw:
      return launch<T, float, false, false, false, kEpiStore, kSchedK>(p, s);
    default:
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm_simt(GemmOp op, int dtype, const GemmParams& p,
                     hipStream_t s) {
  return dtype == MOE_F32 ? dispatch<float>(op, p, s)
                          : dispatch<bf16>(op, p, s);
}

}  // namespace moe
