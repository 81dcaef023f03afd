// Ragged grouped GEMM on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// One workgroup computes a BM x BN output tile (two of them, sharing A, in
// the dual form used by the SwiGLU up-projection). Operand tiles are
// staged in LDS as rows of BK bf16 with the contraction index contiguous,
// in 16-byte chunks whose position is XOR-swizzled with the row so that
// the 128-bit fragment reads of 8 consecutive rows hit distinct banks.
// Operands stored with the row index contiguous are transposed in
// registers, 8x8 at a time, on their way to LDS, so every layout feeds the
// same fragment reads. Two LDS stages: the next k-tile's global loads are
// in flight while the current one feeds the MFMAs.
//
// Tiles come from a device-side list: for row-grouped problems, row tile
// mt maps to (expert, first row) by a binary search in the tile prefix the
// permute step wrote, so no host ever sees the expert loads. The grid is
// sized by the host-known upper bound; surplus workgroups exit at once.
// Workgroup ids are remapped so each XCD gets one contiguous run of
// logical tiles, and logical tiles are ordered n-group-major, then row
// tile, then n within the group, so the ~32 tiles an XCD runs together
// share B panels and A rows in that XCD's L2.
#include "gemm.h"

namespace moe {
namespace {

template <int ROWS, int BK, int NT, bool KC>
struct TileLoader {
  static constexpr int CPR = BK / 8;  // 16-byte chunks per LDS row
  // KC: 16-byte chunks per thread. MC: 8x8 sub-blocks per thread (some
  // threads may have none when the tile is small), 8 chunks each.
  static constexpr int NSUB = (ROWS / 8) * (BK / 8);
  static constexpr int SUBS = (NSUB + NT - 1) / NT;
  static constexpr int NREG = KC ? ROWS * CPR / NT : SUBS * 8;
  static_assert(!KC || (ROWS * CPR) % NT == 0, "tile / thread mismatch");
  u32x4 r[NREG];

  // element (row, k) at base[row * ld + k] (KC) or base[k * ld + row].
  __device__ __forceinline__ void load(const bf16* base, long ld, int row0,
                                       int row_end, int k0, int k_end,
                                       int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int q = tid + i * NT;
        const int row = row0 + q / CPR, k = k0 + (q % CPR) * 8;
        if (row < row_end && k < k_end)
          r[i] = *(const u32x4*)(base + (long)row * ld + k);
        else
          r[i] = u32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        const int q = tid + s * NT;  // sub-block id
        if (NSUB % NT != 0 && q >= NSUB) break;
        const int rb = q % (ROWS / 8), kb = q / (ROWS / 8);
        const int row = row0 + rb * 8;
        u32x4 v[8];
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int k = k0 + kb * 8 + kk;
          if (row < row_end && k < k_end)
            v[kk] = *(const u32x4*)(base + (long)k * ld + row);
          else
            v[kk] = u32x4{0, 0, 0, 0};
        }
        // transpose: out row rr holds k = 0..7 of input column rr
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const uint32_t lo = v[2 * qq][rr / 2], hi = v[2 * qq + 1][rr / 2];
            r[s * 8 + rr][qq] = (rr & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                         : ((lo & 0xffffu) | (hi << 16));
          }
        }
      }
    }
  }

  __device__ __forceinline__ static int slot(int row, int c) {
    return row * CPR + (c ^ (row & (CPR - 1)));
  }

  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NREG; ++i) {
        const int q = tid + i * NT;
        lds[slot(q / CPR, q % CPR)] = r[i];
      }
    } else {
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        const int q = tid + s * NT;
        if (NSUB % NT != 0 && q >= NSUB) break;
        const int rb = q % (ROWS / 8), kb = q / (ROWS / 8);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) lds[slot(rb * 8 + rr, kb)] = r[s * 8 + rr];
      }
    }
  }
};

__device__ __forceinline__ float fast_sigmoid(float a) {
  return 1.0f / (1.0f + __expf(-a));
}

template <int BM, int BN, int BK, int WGM, int WGN, bool A_KC, bool B_KC,
          bool DUAL, int EPI, int SCHED, typename TO>
__global__ __launch_bounds__(WGM * WGN * kWave) void mfma_gemm(GemmParams p) {
  constexpr int NT = WGM * WGN * kWave;
  constexpr int NB_OPS = DUAL ? 2 : 1;
  constexpr int CPR = BK / 8;
  constexpr int WM = BM / WGM, WN = BN / WGN;  // wave tile (per B operand)
  constexpr int MB = WM / 32, NB = WN / 32;    // 32x32 blocks per wave
  constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
  constexpr int STAGE = A_CH + NB_OPS * B_CH;  // 16-byte chunks per stage
  static_assert(MB >= 1 && NB >= 1 && BK % 16 == 0, "tile shape");

  __shared__ u32x4 lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int tiles_n = (p.N + BN - 1) / BN;

  // ---------------------------------------------------------- tile lookup
  int g = 0, m0, m_end, n0, k_beg = 0, k_end = p.K;
  {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    if (SCHED == kSchedM) {
      constexpr int GN = 4;
      const int MT = p.tiles_m_max;
      const int ng = L / (MT * GN);
      const int within = L % (MT * GN);
      const int gsz = min(GN, tiles_n - ng * GN);
      if (gsz <= 0 || within >= MT * gsz) return;
      const int mt = within / gsz;
      n0 = (ng * GN + within % gsz) * BN;
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
      if (L >= p.G * tiles_m * tiles_n) return;
      g = L / (tiles_m * tiles_n);
      const int rem = L % (tiles_m * tiles_n);
      m0 = (rem / tiles_n) * BM;
      n0 = (rem % tiles_n) * BN;
      m_end = p.M;
      k_beg = p.off[g];
      k_end = p.off[g + 1];
    }
  }

  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / WGN, wn = wave % WGN;

  f32x16 acc[NB_OPS][MB][NB];
#pragma unroll
  for (int o = 0; o < NB_OPS; ++o)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[o][i][j] = f32x16{};

  TileLoader<BM, BK, NT, A_KC> la;
  TileLoader<BN, BK, NT, B_KC> lb[NB_OPS];

  const long b_goff = SCHED == kSchedM ? (long)g * p.sB : 0;
  auto issue_loads = [&](int k0) {
    const bf16* A = (const bf16*)p.A;
    const bf16* B0 = (const bf16*)p.B;
    const bf16* B1 = (const bf16*)p.B2;
    int kk = k0, kend = k_end;
    if (k0 >= p.K1) {  // K-concatenation: second operand pair
      A = (const bf16*)p.A2;
      B0 = (const bf16*)p.B2;
      kk = k0 - p.K1;
      kend = k_end - p.K1;
    } else if (!DUAL && p.K1 < k_end) {
      kend = p.K1;
    }
    la.load(A, p.lda, m0, m_end, kk, kend, tid);
    lb[0].load(B0 + b_goff, p.ldb, n0, p.N, kk, kend, tid);
    if (DUAL) lb[NB_OPS - 1].load(B1 + b_goff, p.ldb, n0, p.N, kk, kend, tid);
  };
  auto commit = [&](int stage) {
    u32x4* s = lds + stage * STAGE;
    la.store(s, tid);
    lb[0].store(s + A_CH, tid);
    if (DUAL) lb[NB_OPS - 1].store(s + A_CH + B_CH, tid);
  };

  const int nk = (k_end - k_beg + BK - 1) / BK;
  if (nk > 0) {
    issue_loads(k_beg);
    commit(0);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) issue_loads(k_beg + (kt + 1) * BK);
    const u32x4* sA = lds + cur * STAGE;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks * 2 + lane / 32;
      bf16x8 af[MB], bfr[NB_OPS][NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int row = wm * WM + i * 32 + lane % 32;
        af[i] = __builtin_bit_cast(bf16x8, sA[row * CPR + (c ^ (row & (CPR - 1)))]);
      }
#pragma unroll
      for (int o = 0; o < NB_OPS; ++o)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int row = wn * WN + j * 32 + lane % 32;
          bfr[o][j] = __builtin_bit_cast(
              bf16x8, sA[A_CH + o * B_CH + row * CPR + (c ^ (row & (CPR - 1)))]);
        }
#pragma unroll
      for (int o = 0; o < NB_OPS; ++o)
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[o][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                af[i], bfr[o][j], acc[o][i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) commit(cur ^ 1);
    __syncthreads();
  }

  // -------------------------------------------------------------- epilogue
  // 32x32 accumulator layout: element r of lane l is row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32 of the block.
  TO* C = (TO*)p.C + (SCHED == kSchedK ? (long)g * p.sC : 0);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = n0 + wn * WN + j * 32 + lane % 32;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * WM + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row >= m_end) continue;
        const long o = (long)row * p.ldc + col;
        const float v = acc[0][i][j][r];
        if (EPI == kEpiStore) {
          C[o] = from_f32<TO>(v);
        } else if (EPI == kEpiSwiglu) {
          const float b = acc[NB_OPS - 1][i][j][r];
          if (C) C[o] = from_f32<TO>(v * fast_sigmoid(v) * b);
          if (p.C2) ((TO*)p.C2)[o] = from_f32<TO>(v);
          if (p.C3) ((TO*)p.C3)[o] = from_f32<TO>(b);
        } else {
          const float a = to_f32(((const bf16*)p.aux_a)[o]);
          const float b = to_f32(((const bf16*)p.aux_b)[o]);
          const float s = fast_sigmoid(a);
          C[o] = from_f32<TO>(v * b * s * (1.0f + a * (1.0f - s)));
          ((TO*)p.C2)[o] = from_f32<TO>(v * a * s);
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, bool A_KC, bool B_KC,
          bool DUAL, int EPI, int SCHED, typename TO>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  const long tiles_n = (p.N + BN - 1) / BN;
  long tiles;
  if (SCHED == kSchedM) {
    const long ngroups = (tiles_n + 3) / 4;
    tiles = ngroups * p.tiles_m_max * 4;
  } else {
    tiles = (long)p.G * ((p.M + BM - 1) / BM) * tiles_n;
  }
  if (tiles <= 0) return hipSuccess;
  tiles = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
  if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(
      (mfma_gemm<BM, BN, BK, WGM, WGN, A_KC, B_KC, DUAL, EPI, SCHED, TO>),
      dim3((unsigned)tiles), dim3(WGM * WGN * kWave), 0, s, p);
  return hipGetLastError();
}

// Large tiles: 256 x 256 outputs (256 x 128 per B in the dual form),
// 4 waves of 128 x 128 (128 x 64 x 2). Small tiles: 128 x 128 (128 x 64).
template <bool A_KC, bool B_KC, bool DUAL, int EPI, int SCHED, typename TO>
hipError_t launch_sized(bool big, const GemmParams& p, hipStream_t s) {
  if (big)
    return launch<256, DUAL ? 128 : 256, 64, 2, 2, A_KC, B_KC, DUAL, EPI,
                  SCHED, TO>(p, s);
  return launch<128, DUAL ? 64 : 128, 64, 2, 2, A_KC, B_KC, DUAL, EPI, SCHED,
                TO>(p, s);
}

}  // namespace

bool mfma_supported(GemmOp op, const GemmParams& p) {
  // 16-byte chunk loads need K (and K1) in multiples of 8; the k-tile of
  // a K-concatenation must not straddle the seam; transposed (row
  // contiguous) operands are loaded 8 rows at a time.
  if (p.K % 8) return false;
  if (op == kOpDgrad1 && p.K1 % 64) return false;
  if ((op == kOpDgrad2 || op == kOpDgrad1) && p.N % 8) return false;
  if (op == kOpWgrad && (p.M % 8 || p.N % 8)) return false;
  return true;
}

hipError_t gemm_mfma(GemmOp op, GemmParams p,
                     const int32_t* const* tile_off_by_bm, hipStream_t s) {
  if (!mfma_supported(op, p)) return hipErrorNotSupported;
  // Big tiles when the average group has enough rows to fill them.
  bool big;
  if (op == kOpWgrad) {
    big = p.M >= 256 && p.N >= 256;
  } else {
    const long rows_per_group = p.off ? (long)p.M / (p.G > 0 ? p.G : 1) : p.M;
    big = rows_per_group >= 192 && p.N >= 256;
    if (op == kOpRouter) big = false;
    const int bm = big ? 256 : 128;
    if (p.off) {
      p.tile_off = tile_off_by_bm[tile_bm_slot(bm)];
      p.tiles_m_max = (p.M + bm - 1) / bm + (p.G < p.M ? p.G : p.M);
    } else {
      p.tiles_m_max = (p.M + bm - 1) / bm;
    }
  }
  switch (op) {
    case kOpRouter:
      return launch_sized<true, true, false, kEpiStore, kSchedM, float>(big, p, s);
    case kOpGemm1:
      return launch_sized<true, true, true, kEpiSwiglu, kSchedM, bf16>(big, p, s);
    case kOpGemm2:
      return launch_sized<true, true, false, kEpiStore, kSchedM, bf16>(big, p, s);
    case kOpDgrad2:
      return launch_sized<true, false, false, kEpiSwigluBwd, kSchedM, bf16>(big, p, s);
    case kOpDgrad1:
      return launch_sized<true, false, false, kEpiStore, kSchedM, bf16>(big, p, s);
    case kOpWgrad:
      return launch_sized<false, false, false, kEpiStore, kSchedK, bf16>(big, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
