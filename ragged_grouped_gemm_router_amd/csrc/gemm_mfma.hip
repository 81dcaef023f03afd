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
#include <climits>
#include <cstdlib>
#include <cstring>
#include <type_traits>
#include <utility>

#include "gemm.h"
#include "mx.h"
#include "tile_map.h"

namespace moe {
namespace {

// LDS position of 16-byte chunk c in a tile row of CPR chunks. The LDS of
// gfx950 has 64 banks of 4 bytes, so a 128-bit read serves 16 lanes per
// pass; those lanes read the same logical chunk of 16 consecutive rows,
// which lie two (CPR = 8) or four (CPR = 4) to a 256-byte bank line. The
// XOR with the row's line index gives each of them its own 16-byte bank
// group.
template <int CPR>
__device__ __forceinline__ int swz(int row, int c) {
  if constexpr (CPR == 8) return c ^ ((row >> 1) & 7);
  else return c ^ ((row >> 2) & 3);
}

// Raw (untyped, unswizzled) buffer resource starting at `base`, with the
// range check at its 4 GiB maximum: the DMA loads below address it with a
// per-lane offset plus a scalar k offset, both far smaller than that.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kBufWord3 = 0x00020000;
__device__ __forceinline__ Rsrc make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1,
                                           kBufWord3);
}
// Resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ Rsrc make_rsrc_n(const void* base, long bytes) {
  const long n = bytes < 0 ? 0 : (bytes > 0x7fffffffL ? 0x7fffffffL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n,
                                           kBufWord3);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
// ds_read_b64_tr_b16 (lane layout: see the k-major B of the direct-to-LDS
// kernel). The restrict qualifier gives the inlined read alias-scope
// metadata, as a plain LDS load carries type-based alias metadata; without
// it the compiler's wait insertion makes every such read wait for all LDS
// DMA in flight (vmcnt(0)), which drains the prefetch of the next k-tiles.
// The kernels order their DMA and fragment reads with explicit waits (the
// tile barrier).
__device__ __forceinline__ s16x4 lds_read_tr16(const char* __restrict__ a) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)a);
}
// 16 bytes per lane from r + voff + soff into LDS at dst + 16 * lane. (A
// plain function: called straight from a kernel template, the builtin
// keeps clang's host pass from emitting that kernel's launch stub.)
// f(std::integral_constant<int, i>{}) for i = 0 .. N-1 in order: a loop
// whose index is a constant expression in the body
template <typename Fn, int... I>
__device__ __forceinline__ void static_for_seq(Fn&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// Tile barrier of the direct-to-LDS kernels: this wave's LDS reads are
// complete and at most N of its loads are outstanding (vmcnt N, lgkmcnt 0),
// then all waves meet. Loads complete in issue order, so N = the loads
// issued after the newest ones the next stage needs. Before the barrier
// only a compiler barrier keeps LDS accesses in place: a release fence
// would also wait for every DMA write to LDS (vmcnt 0), including the
// newest ones left in flight on purpose, into a stage no wave reads before
// a later barrier. The acquire fence keeps later LDS reads below it.
template <int N>
__device__ __forceinline__ void tile_barrier() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void dma16(Rsrc r, char* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

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
    return row * CPR + swz<CPR>(row, c);
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

// sigmoid of the SwiGLU epilogues: hardware exp2 and reciprocal (about 1
// ulp each), far inside the bf16 rounding of the stored result, instead of
// an IEEE division (ten instructions per element in an epilogue that no
// other work overlaps: one workgroup per CU)
__device__ __forceinline__ float fast_sigmoid(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// This workgroup's output tile (the decode and its order are described
// with decode_tile); false for surplus workgroups.
template <int BM, int BN, int SCHED, int TAIL = 0>
__device__ __forceinline__ bool lookup_tile(const GemmParams& p, Tile& t) {
  return decode_tile<BM, BN, SCHED, TAIL>(p, (int)blockIdx.x, (int)gridDim.x, t);
}

// Tile output through LDS: the fp32 values of the wave's 32x32 blocks
// (value(i, j, r) for accumulator element r of block (i, j)) go to LDS as
// rows of the tile, ROWS at a time, and every thread then hands
// store(row, col, v[8]) eight consecutive columns of one row, so global
// traffic moves in 16-byte row-contiguous pieces instead of 2-byte
// scattered ones. The row pitch is padded by 8 floats so that the two
// half-waves' stores (rows 4 apart) use disjoint banks. The caller has
// finished reading LDS for operands; the LDS is free on return.
template <int BM, int BN, int WM, int WN, int MB, int NB, int NT, int ROWS,
          int PW = 8>
struct StageOut {
  static constexpr int PITCH = BN + 8;
  static constexpr int BYTES = ROWS * PITCH * 4;
  static_assert(BM % ROWS == 0, "pass rows");
  static_assert(PW % 8 == 0 && BN % PW == 0, "piece width");

  // rows: the tile's rows that are stored (a workgroup-uniform count);
  // passes wholly past them are skipped, since every store there would
  // be masked (a ragged group's tile that ends in its first pass)
  template <typename V, typename St>
  __device__ __forceinline__ static void run(char* lds, int wm, int wn,
                                             int lane, V value, St store,
                                             int rows) {
    float* st = (float*)lds;
    const int tid = threadIdx.x;
#pragma unroll
    for (int pass = 0; pass < BM / ROWS; ++pass) {
      const int r0 = pass * ROWS;
      if (r0 >= rows) break;
      __syncthreads();  // LDS free (operands read, or previous pass out)
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int rb = wm * WM + i * 32;  // block's first tile row
        if (rb + 32 <= r0 || rb >= r0 + ROWS) continue;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int col = wn * WN + j * 32 + lane % 32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = rb + 8 * (r / 4) + 4 * (lane / 32) + r % 4 - r0;
            st[row * PITCH + col] = value(i, j, r);
          }
        }
      }
      __syncthreads();
      const int CH = min(ROWS, rows - r0) * (BN / PW);
#pragma unroll 2
      for (int c = tid; c < CH; c += NT) {
        const int row = c / (BN / PW), col = (c % (BN / PW)) * PW;
        float v[PW];
#pragma unroll
        for (int q = 0; q < PW; q += 4) {
          const f32x4 x = *(const f32x4*)(st + row * PITCH + col + q);
          v[q] = x[0];
          v[q + 1] = x[1];
          v[q + 2] = x[2];
          v[q + 3] = x[3];
        }
        store(r0 + row, col, v);
      }
    }
    __syncthreads();
  }
};

__device__ __forceinline__ bf16x8 pack8(const float* v) {
  bf16x8 o;
#pragma unroll
  for (int q = 0; q < 8; ++q) o[q] = (bf16)v[q];
  return o;
}

// 32x32 accumulator layout: element r of lane l is row
// 8*(r/4) + 4*(l/32) + r%4, column l%32 of the block.
template <int WM, int WN, int MB, int NB, int NB_OPS, int EPI, int SCHED,
          typename TO>
__device__ __forceinline__ void epilogue(const GemmParams& p, const Tile& t,
                                         f32x16 (&acc)[NB_OPS][MB][NB],
                                         int wm, int wn, int lane) {
  TO* C = (TO*)p.C + (SCHED == kSchedK ? (long)t.g * p.sC : 0);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int col = t.n0 + wn * WN + j * 32 + lane % 32;
      if (col >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = t.m0 + wm * WM + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        if (row >= t.m_end) continue;
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

// ---------------------------------------------------------------------------
// Register-staged kernel: any operand layout (used where an operand is
// stored with its row index contiguous, i.e. the backward products).
// ---------------------------------------------------------------------------
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
  Tile t;
  if (!lookup_tile<BM, BN, SCHED>(p, t)) return;
  const int m0 = t.m0, m_end = t.m_end, n0 = t.n0, k_beg = t.k_beg,
            k_end = t.k_end;

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

  const long b_goff = SCHED == kSchedM ? (long)t.g * p.sB : 0;
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
        af[i] = __builtin_bit_cast(bf16x8, sA[row * CPR + swz<CPR>(row, c)]);
      }
#pragma unroll
      for (int o = 0; o < NB_OPS; ++o)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int row = wn * WN + j * 32 + lane % 32;
          bfr[o][j] = __builtin_bit_cast(
              bf16x8, sA[A_CH + o * B_CH + row * CPR + swz<CPR>(row, c)]);
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
  epilogue<WM, WN, MB, NB, NB_OPS, EPI, SCHED, TO>(p, t, acc, wm, wn, lane);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel for k-contiguous operands (the forward products).
//
// global_load_lds_dwordx4 moves 16 bytes per lane from HBM straight into
// LDS: lane l of a wave writes LDS bytes [base + 16 l, base + 16 l + 16),
// so one instruction fills 1 KB = RPI rows of the tile. Each lane fetches
// the global chunk that belongs at its LDS position under the XOR
// swizzle, so the operands need no registers on their way in and there is
// no LDS-write phase. S stages form a ring: the loads for k-tile kt+S-1 are
// issued right after the barrier that ends the use of its stage, S-1
// tiles ahead of the MFMAs that consume them. Rows past the group's end
// (and columns past N) are fetched from the last valid row: their
// products land only in outputs the epilogue discards. K must be a
// multiple of BK.
// ---------------------------------------------------------------------------

// Fragment read order of a k-substep: the order in which its MFMAs, q =
// (o * MB + i) * NB + j taking A block i and B block (o, j), first use
// them (FIRST_USE), else A blocks then B blocks. Index r < MB is A block r,
// else B block (r - MB) / NB, (r - MB) % NB.
template <int MB, int NB, int NOPS, bool FIRST_USE>
struct ReadOrder {
  int r[MB + NOPS * NB];
  constexpr ReadOrder() : r{} {
    bool seen[MB + NOPS * NB] = {};
    int n = 0;
    if (!FIRST_USE) {
      for (; n < MB + NOPS * NB; ++n) r[n] = n;
      return;
    }
    for (int q = 0; q < NOPS * MB * NB; ++q) {
      const int ra = (q / NB) % MB, rb = MB + q / (MB * NB) * NB + q % NB;
      if (!seen[rb]) seen[rb] = true, r[n++] = rb;
      if (!seen[ra]) seen[ra] = true, r[n++] = ra;
    }
  }
};

// Operand formats of the direct-to-LDS kernel.
//   bf16 : v_mfma_f32_32x32x16_bf16, 8 bf16 per lane per fragment
//   MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3, 32 bytes per lane per
//          fragment = one 32-element MX block of the lane's row, with that
//          block's E8M0 scale passed per lane
template <bool MX> struct Fmt;
template <> struct Fmt<false> {
  static constexpr int ES = 2, KSTEP = 16, FC = 1;
  typedef bf16x8 Frag;
};
template <> struct Fmt<true> {
  static constexpr int ES = 1, KSTEP = 64, FC = 2;
  typedef int32_t Frag __attribute__((ext_vector_type(8)));
};

template <int BM, int BN, int S, int WGM, int WGN, bool DUAL, int EPI,
          typename TO, bool MX, int SCHED = kSchedM, int TAIL = 0,
          int SKIP = 0, bool KCAT = false, int SB = 0, bool BKM = false>
__global__ __launch_bounds__(WGM * WGN * kWave) void mfma_gemm_dl(GemmParams p) {
  using F = Fmt<MX>;
  typedef typename F::Frag Frag;
  constexpr int NW = WGM * WGN;
  constexpr int NB_OPS = DUAL ? 2 : 1;
  constexpr int RB = 128;            // bytes of one tile row per k-tile
  constexpr int BK = RB / F::ES;     // k-tile in elements
  constexpr int KS = BK / F::KSTEP;  // MFMA k-substeps per k-tile
  constexpr int CPR = RB / 16;       // 16-byte chunks per tile row
  constexpr int RPI = 64 / CPR;      // rows per 1 KB wave instruction
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  constexpr int STAGE = A_BYTES + NB_OPS * B_BYTES;
  constexpr int A_INS = BM / RPI / NW, B_INS = BN / RPI / NW;
  // SB > S: the B operands run in a ring of SB stages of their own, so a
  // weight-streaming product keeps SB - 1 k-tiles of B in flight while A
  // (re-read by every column tile, so mostly an L2 hit) keeps S - 1
  constexpr bool RING_B = SB > S;
  constexpr int S_B = RING_B ? SB : S;
  constexpr int A_STRIDE = RING_B ? A_BYTES : STAGE;
  constexpr int B_STRIDE = RING_B ? NB_OPS * B_BYTES : STAGE;
  constexpr int B_BASE = RING_B ? S * A_BYTES : A_BYTES;
  constexpr int RING_BYTES = RING_B ? S * A_BYTES + SB * NB_OPS * B_BYTES : S * STAGE;
  constexpr int NBL = NB_OPS * B_INS;  // B DMA instructions per k-tile
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "tile shape");
  static_assert(MB >= 1 && NB >= 1, "tile shape");
  static_assert(S >= 2 && KS % 2 == 0, "stage count, even substep count");
  static_assert((S - 1) * (A_INS + NBL) + (S_B - S) * NBL + (MX ? MB + NB_OPS * NB : 0) <= 63,
                "vmcnt range");
  // The tile barrier's wait leaves the newest (S_B - S) * NBL loads in
  // flight. Only NBL B loads of one k-tile follow the A loads of tile
  // kt + 1 in issue order, so that count covers no A load only when the B
  // ring is exactly one stage deeper than A's.
  static_assert(!RING_B || SB == S + 1, "B ring depth must be S + 1");
  // BKM: B stored k-major, element (n, k) of a group at B[k * ldb + n] (the
  // weights of the data-gradient products, read as the forward stores
  // them). A k-tile is DMA'd as it lies: BK k-rows of BN elements, the
  // 16-byte chunk c of k-row k at position c ^ (4 * (k & 3)), CPK chunks
  // per k-row and KPI k-rows per 1 KB wave instruction, the same
  // instruction count as the row-major form. A fragment (32 columns x 16 k)
  // is two ds_read_b64_tr_b16: within each 16-lane group, lane j points at
  // k-row kb + j / 4, columns c0 + 4 (j % 4) .. +3, and the read hands lane
  // i the four k values kb .. kb + 3 of column c0 + i. Rows kb .. kb + 3
  // then sit in distinct quarters of the 64 banks: conflict-free.
  static_assert(!BKM || (!MX && !DUAL && SCHED == kSchedM && BN % 128 == 0 &&
                         BN <= 512), "k-major B");
  constexpr int CPK = BN / 8, KPI = BKM ? 64 / CPK : 1;

  // the epilogue stages 128 rows at a time (the quantising one only for
  // the optional pre-activation copies)
  constexpr int kEpiRows = BM > 128 ? 128 : BM;
  constexpr int EPI_BYTES =
      StageOut<BM, BN, WM, WN, MB, NB, NW * kWave, kEpiRows>::BYTES;
  // TACC: the bf16-output products other than the quantising one take the
  // MFMA operands swapped and accumulate C^T (element r of lane l: row
  // l % 32, column 8 (r / 4) + 4 (l / 32) + r % 4 of the 32 x 32 block), so
  // the epilogue hands 8-column row pieces straight from registers to the
  // stores after one swap of lane halves per pair of register quads, with
  // no LDS staging and no barrier. Not the 4-wave big tile (it would
  // spill), and not the SwiGLU backward, whose loads of the saved a and b
  // would come in 32-byte row pieces instead of whole rows (dgrad2 13%
  // slower on the Mixtral shape)
  constexpr bool TACC = !MX && sizeof(TO) == 2 && EPI != kEpiSwigluMx &&
                        EPI != kEpiSwigluBwd && !(NW == 4 && BM == 256);
  __shared__ __attribute__((aligned(1024))) char
      lds[TACC || RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES];

  // the tile; grouped contraction (SCHED K): k-tiles [kt0, kt0 + nk) of
  // the group's range, which the host pads to whole k-tiles
  Tile t;
  if (!lookup_tile<BM, BN, SCHED, TAIL>(p, t)) return;
  const int kt0 = SCHED == kSchedK ? t.k_beg / BK : 0;
  const int nk = SCHED == kSchedK ? (t.k_end - t.k_beg) / BK : p.K / BK;
  const int tid = threadIdx.x, lane = tid % kWave;
  // wave-uniform, so every LDS destination below is a scalar (M0) value
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WGN, wn = wave % WGN;
  static_assert(CPR == 8, "128-byte tile rows");

  // DMA sources: buffer resources based at the tile's first row, so the
  // per-lane offsets stay small at any problem size and the k-tile offset
  // rides in the scalar offset; each lane fetches the 16-byte chunk that
  // belongs at its (swizzled) LDS position.
  // Gathered A: the resource spans the whole source matrix and each lane's
  // offset is its row's source row (the host keeps it below 2^31 bytes).
  const int r_in = lane / CPR, phys = lane % CPR;
  const bool gather = p.gsrc != nullptr;
  const Rsrc ra = make_rsrc((const char*)p.A +
                            (gather ? 0 : (long)t.m0 * p.lda * F::ES));
  int a_off[A_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int row = (j * NW + wave) * RPI + r_in;
    const int grow = min(t.m0 + row, t.m_end - 1);
    const int src = gather ? p.gsrc[grow] / p.gdiv : grow - t.m0;
    a_off[j] = src * (int)p.lda * F::ES + swz<CPR>(row, phys) * 16;
  }
  // (k-major B: based at the tile's first column; a lane's chunk past
  // column N is clamped to the last in-range one, its data reaching only
  // output columns past N)
  const long b_base = (long)t.g * p.sB + (BKM ? (long)t.n0 : (long)t.n0 * p.ldb);
  Rsrc rb[NB_OPS];
  rb[0] = make_rsrc((const char*)p.B + b_base * F::ES);
  if (DUAL) rb[NB_OPS - 1] = make_rsrc((const char*)p.B2 + b_base * F::ES);
  int b_off[B_INS];
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    if constexpr (BKM) {
      const int kr = (j * NW + wave) * KPI + lane / CPK;
      const int c = (lane % CPK) ^ (4 * (kr & 3));
      b_off[j] = kr * p.ldb * 2 + min(c * 8, p.N - t.n0 - 8) * 2;
    } else {
      const int row = (j * NW + wave) * RPI + r_in;
      const int grow = min(t.n0 + row, p.N - 1);
      b_off[j] = (grow - t.n0) * p.ldb * F::ES + swz<CPR>(row, phys) * 16;
    }
  }
  // KCAT: the contraction runs over [A | A2] . [B ; B2], the first K1
  // indices from A, B (k-tiles below nk1) and the rest from A2, B2, all
  // with the same strides, so the lane offsets serve both parts
  static_assert(!KCAT || (!DUAL && !MX && SCHED == kSchedM), "K-concatenation");
  const int nk1 = KCAT ? p.K1 / BK : 0;
  Rsrc ra2 = ra, rb2 = rb[0];
  if (KCAT) {
    ra2 = make_rsrc((const char*)p.A2 + (long)t.m0 * p.lda * F::ES);
    rb2 = make_rsrc((const char*)p.B2 + b_base * F::ES);
  }

  // DMA instruction d of a k-tile (d < A_INS: operand A of k-tile kt
  // into A stage sa, then each B of k-tile ktb into B stage sbs)
  auto issue_one = [&](int kt, int sa, int ktb, int sbs, int d) {
    if (d < A_INS) {
      const bool second = KCAT && kt >= nk1;
      const int k0 = (kt0 + kt - (second ? nk1 : 0)) * RB;
      dma16(second ? ra2 : ra, lds + sa * A_STRIDE + (d * NW + wave) * 1024,
            a_off[d], k0);
    } else {
      const bool second = KCAT && ktb >= nk1;
      // byte offset of the k-tile: along the row, or BK k-rows down
      const int k0 = (kt0 + ktb - (second ? nk1 : 0)) * (BKM ? BK * p.ldb * 2 : RB);
      const int o = (d - A_INS) / B_INS, j = (d - A_INS) % B_INS;
      dma16(second ? rb2 : rb[o],
            lds + B_BASE + sbs * B_STRIDE + o * B_BYTES + (j * NW + wave) * 1024,
            b_off[j], k0);
    }
  };

  // MXFP8: in the span-grouped scale arrays a row's 4 E8M0 codes for one
  // k-tile are one aligned word and the words of consecutive rows are
  // contiguous, so the 32 rows of a block read one 128-byte line. Each
  // lane reads the words of its row of every block through buffer loads:
  // one resource per operand, the row's byte offset per block in a VGPR
  // (rows past the tile's end clamped, as for the data; B's rows counted
  // in the stacked groups) and the k-tile's span as the scalar offset. They are loaded
  // a tile ahead (s_nxt) and swapped in at the tile barrier.
  constexpr int NSC = MX ? MB + NB_OPS * NB : 1;
  int sa_off[MX ? MB : 1], sb_off[MX ? NB : 1];
  Rsrc rsa = ra, rsb[NB_OPS];
  const int rows_b = p.off ? p.G * p.N : p.N;  // rows of B's scale array
  uint32_t s_cur[NSC], s_nxt[NSC];
  if constexpr (MX) {
    rsa = make_rsrc(p.As);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int row = min(t.m0 + wm * WM + i * 32 + lane % 32, t.m_end - 1);
      sa_off[i] = (gather ? p.gsrc[row] / p.gdiv : row) * 4;
    }
#pragma unroll
    for (int o = 0; o < NB_OPS; ++o)
      rsb[o] = make_rsrc(o ? p.B2s : p.Bs);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      sb_off[j] = (t.g * p.N + min(t.n0 + wn * WN + j * 32 + lane % 32, p.N - 1)) * 4;
  }
  auto load_scales = [&](uint32_t* dst, int kt) {
    if constexpr (MX) {
      const int span = kt0 + kt;
#pragma unroll
      for (int i = 0; i < MB; ++i)
        dst[i] = __builtin_amdgcn_raw_buffer_load_b32(
            rsa, sa_off[i], span * (int)p.s_rows * 4, 0);
#pragma unroll
      for (int o = 0; o < NB_OPS; ++o)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          dst[MB + o * NB + j] = __builtin_amdgcn_raw_buffer_load_b32(
              rsb[o], sb_off[j], span * rows_b * 4, 0);
    }
  };
  f32x16 acc[NB_OPS][MB][NB];
#pragma unroll
  for (int o = 0; o < NB_OPS; ++o)
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[o][i][j] = f32x16{};

  // fragments of one k-substep
  struct Frags {
    Frag a[MB], b[NB_OPS][NB];
  };
  constexpr int N_READ = MB + NB_OPS * NB;        // fragment reads per substep
  constexpr int N_MFMA = NB_OPS * MB * NB;        // MFMAs per substep
  constexpr int N_LOAD = A_INS + NB_OPS * B_INS;  // DMA instructions per k-tile
  // Fragment rows differ from the lane's first row by multiples of 32, so
  // they share its swizzle: the chunk position depends on the lane and the
  // substep only, and the block offset is an immediate of the LDS read.
  const int lrow = lane % 32, half = lane / 32, sw = swz<CPR>(lrow, 0);
  const int a_row0 = (wm * WM + lrow) * RB;
  const int b_row0 = (wn * WN + lrow) * RB;
  // k-major B: the lane's byte offset in the stage for block j at substep
  // 0 (the substep and the second read add k-row multiples, immediates)
  int bkm_off[BKM ? NB : 1];
  if constexpr (BKM) {
    const int grp = lane / 16, gj = lane % 16;
    const int kl = 8 * (grp >> 1) + (gj >> 2);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int c = wn * WN + j * 32 + 16 * (grp & 1) + 4 * (gj & 3);
      bkm_off[j] = kl * (BN * 2) + (((c >> 3) ^ (4 * (kl & 3))) * 16) + (c & 7) * 2;
    }
  }
  auto read_bkm = [&](const char* sbo, int j, int ks) {
    Frag f{};
    if constexpr (BKM) {
      const char* q = sbo + bkm_off[j] + ks * 16 * (BN * 2);
      const s16x4 v0 = lds_read_tr16(q), v1 = lds_read_tr16(q + 4 * (BN * 2));
      typedef short s16x8 __attribute__((ext_vector_type(8)));
      const s16x8 w = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      f = __builtin_bit_cast(Frag, w);
    }
    return f;
  };
  auto read_frag = [&](const char* rowp, int ks) {
    if constexpr (MX) {
      // The scaled MFMA takes bytes 0-15 of a lane from the substep's first
      // 32-element block and bytes 16-31 from its second; half-wave h holds
      // the h-th 16 elements of each block (chunks 4 ks + h and 4 ks + 2 + h
      // of the 128-byte row), matching the per-lane scales of block
      // 2 ks + h of lanes h*32 + row.
      const int c_lo = ks * 4 + half, c_hi = c_lo + 2;
      const u32x4 lo = *(const u32x4*)(rowp + (c_lo ^ sw) * 16);
      const u32x4 hi = *(const u32x4*)(rowp + (c_hi ^ sw) * 16);
      return Frag{(int32_t)lo[0], (int32_t)lo[1], (int32_t)lo[2], (int32_t)lo[3],
                  (int32_t)hi[0], (int32_t)hi[1], (int32_t)hi[2], (int32_t)hi[3]};
    } else {
      return *(const Frag*)(rowp + ((ks * 2 + half) ^ sw) * 16);
    }
  };
  // Fragment reads follow the order in which the MFMAs of the substep
  // first use them (MFMA q takes A block i and B block (o, j)), so the
  // first MFMAs of a region wait only for the first reads of the region
  // before it. The dual MXFP8 tile keeps A-then-B order: its longer-lived
  // 32-byte fragments would spill.
  constexpr ReadOrder<MB, NB, NB_OPS, !(MX && DUAL)> kOrder{};
  // fragment kOrder.r[m] of substep ks (r < MB: A block r, else B block)
  // from the A stage at sa and the B stage at sbb
  auto read_one = [&](const char* sa, const char* sbb, int ks, Frags& f, int m) {
    const int r = kOrder.r[m];
    if (r < MB) {
      f.a[r] = read_frag(sa + a_row0 + r * 32 * RB, ks);
    } else {
      const int o = (r - MB) / NB, j = (r - MB) % NB;
      if constexpr (BKM)
        f.b[o][j] = read_bkm(sbb + o * B_BYTES, j, ks);
      else
        f.b[o][j] = read_frag(sbb + b_row0 + o * B_BYTES + j * 32 * RB, ks);
    }
  };
  // per-lane E8M0 scale operands of one substep: block ks*2 + lane/32
  uint32_t sc[NSC];
  auto substep_scales = [&](int ks) {
    if constexpr (MX) {
      const int sh = 8 * (ks * 2 + lane / 32);
#pragma unroll
      for (int q = 0; q < NSC; ++q) sc[q] = (s_cur[q] >> sh) & 0xffu;
    }
  };
  // SKIP: 32-row blocks of this wave that hold rows of the group: a
  // ragged row tile skips the MFMAs of blocks wholly past the group's end
  // (their rows would be clamped copies, never stored); loads and barriers
  // run unchanged, so every wait count stays exact. SKIP 1: one copy of
  // the k-loop, with a branch per MFMA (groups of about half a tile, where
  // every tile is ragged). SKIP 2 (large groups, most tiles full): the
  // k-loop is compiled twice and a wave whose blocks all hold rows runs the
  // copy without the branches; the dual MXFP8 tile keeps one copy (two
  // spill). A 4-wave tile, 256 accumulator registers, would spill with the
  // branches.
  constexpr bool kSkipTail = SKIP != 0 && SCHED == kSchedM && N_MFMA * 16 <= 128;
  const int act_mb = __builtin_amdgcn_readfirstlane(
      min(MB, max(0, (t.m_end - t.m0 - wm * WM + 31) / 32)));
  // MFMA q of a substep, q = (o * MB + i) * NB + j; sk: the skipping copy
  auto mfma_one = [&](const Frags& f, int q, auto sk) {
    const int o = q / (MB * NB), i = (q / NB) % MB, j = q % NB;
    if (decltype(sk)::value && i >= act_mb) return;
    if constexpr (MX) {
      acc[o][i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.a[i], f.b[o][j], acc[o][i][j], 0, 0, 0, (int)sc[i], 0,
          (int)sc[MB + o * NB + j]);
    } else if constexpr (TACC) {
      acc[o][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          f.b[o][j], f.a[i], acc[o][i][j], 0, 0, 0);
    } else {
      acc[o][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          f.a[i], f.b[o][j], acc[o][i][j], 0, 0, 0);
    }
  };

  auto barrier_after = [&](auto vm_left) {
    tile_barrier<decltype(vm_left)::value>();
  };

  // Prologue: (scales of k-tile 0,) k-tiles 0 .. S-1 in flight, and the
  // B operands of k-tiles S .. S_B-1 (past the last tile, the last one
  // again, into stages nobody reads); wait for tile 0. MXFP8 scales of the
  // dual products run one tile ahead: those of tile kt+1 are issued at the
  // start of tile kt, ahead of that tile's DMA, so the tile barrier's own
  // wait covers them and their copy into s_cur after it waits for nothing.
  // The single-B products with a deeper B ring (SC2) issue them two tiles
  // ahead, right after the barrier, so that the B DMA of tile kt+2 is
  // still the newest load at the next barrier: the compiler then rotates
  // them through a third register set and waits for loads a few MFMAs old
  // at its copy, which costs the dual tile 1-5% of GEMM 1 and the
  // single-B one nothing.
  constexpr bool SC2 = MX && RING_B && !DUAL;
  constexpr int NSC_RING = SC2 ? NSC : 0;
  // SPREAD (B ring one stage deeper than A's): the B DMA of k-tile
  // kt + S_B - 1 goes into the B stage that tile kt - 1 used, free since the
  // barrier that ended tile kt - 1, and is spread over the regions of
  // substeps 0 .. KS-2 of tile kt; the region after a tile barrier then
  // issues only A's DMA, half the burst (a whole k-tile's DMA at once
  // outruns the CU's load path, and both waves of a SIMD stall behind it).
  // The barrier's wait is unchanged: the newest NBL loads at the end of
  // tile kt are still B's, of k-tile kt + S_B - 1.
  constexpr bool SPREAD = RING_B;
  if (nk > 0) {  // (an empty group's tile writes zeros)
  load_scales(SC2 ? s_cur : s_nxt, 0);
#pragma unroll
  for (int i = 0; i < S; ++i)
#pragma unroll
    for (int d = 0; d < N_LOAD; ++d)
      issue_one(min(i, nk - 1), i, min(i, nk - 1), i, d);
  if constexpr (SC2) load_scales(s_nxt, min(1, nk - 1));
  if constexpr (!SPREAD) {
#pragma unroll
    for (int i = S; i < S_B; ++i)
#pragma unroll
      for (int d = A_INS; d < N_LOAD; ++d) issue_one(0, 0, min(i, nk - 1), i, d);
  }
  barrier_after(std::integral_constant<int, (S - 1) * N_LOAD + NSC_RING +
                                                (SPREAD ? 0 : (S_B - S) * NBL)>{});
  if constexpr (MX && !SC2) {
#pragma unroll
    for (int q = 0; q < NSC; ++q) s_cur[q] = s_nxt[q];
  }
  Frags fa, fb;
#pragma unroll
  for (int r = 0; r < N_READ; ++r) read_one(lds, lds + B_BASE, 0, fa, r);

  // One region per k-substep. The MFMAs run on fragments read a region
  // earlier; the memory instructions of the region (the next substep's
  // fragment reads and, at the last substep of a k-tile, the DMA of k-tile
  // kt+S into the stage tile kt used) sit between them, at most a few per
  // MFMA, so the in-order issue of a long memory burst never leaves the
  // matrix pipe idle. The tile barrier waits until only the S-2 newest
  // tiles' DMA (and, with a deeper B ring, the B DMA of the S_B-S newest
  // B tiles) is outstanding, i.e. for tile kt+1. The first H MFMAs
  // precede every new read: their wait for the current fragments then
  // covers no read issued here. Every step is fenced with sched_barrier to
  // keep this order. (MXFP8: the next tile's scales are fetched in the
  // first region and swapped in after the tile barrier, once their wait is
  // free.)
  constexpr int H = N_MFMA >= 8 ? 2 : N_MFMA >= 2 ? 1 : 0;
#define MOE_FENCE() __builtin_amdgcn_sched_barrier(0)
  auto kloop = [&](auto sk) {
  // stage of k-tile kt (kt mod S) and of k-tile kt + 1, kept as counters
  int st = 0, st_next = S > 1 ? 1 : 0;
  int sbt = 0, sbt_next = 1;  // the same for the B ring
  int sbt_prev = S_B - 1;     // B stage of k-tile kt - 1
  for (int kt = 0; kt < nk; ++kt) {
    const char* sa = lds + st * A_STRIDE;
    const char* sa_next = lds + st_next * A_STRIDE;
    const char* sbb = lds + B_BASE + sbt * B_STRIDE;
    const char* sbb_next = lds + B_BASE + sbt_next * B_STRIDE;
    static_for<KS>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      Frags& cur = (ks & 1) ? fb : fa;
      Frags& nxt = (ks & 1) ? fa : fb;
      constexpr bool last = ks + 1 == KS;
      // memory ops of this region: N_READ reads and the DMA instructions
      // [d_lo, d_hi) of a k-tile (all N_LOAD at the last substep, or with
      // SPREAD A's there and a share of B's at each earlier substep)
      constexpr int NM_MAX = N_READ + N_LOAD;
      constexpr int d_lo = !SPREAD || last ? 0 : A_INS + ks * NBL / (KS - 1);
      constexpr int d_hi = !SPREAD ? (last ? N_LOAD : 0)
                           : last  ? A_INS
                                   : A_INS + (ks + 1) * NBL / (KS - 1);
      constexpr int nm = N_READ + d_hi - d_lo;
      substep_scales(ks);
      MOE_FENCE();
#pragma unroll
      for (int q = 0; q < H; ++q) mfma_one(cur, q, sk);
      MOE_FENCE();
      if constexpr (ks == 0 && MX && !SC2) {
        load_scales(s_nxt, min(kt + 1, nk - 1));
        MOE_FENCE();
      }
      if constexpr (last) {
        // Branch-free so the wait counters stay exact: past the last tile
        // the reads return unused data and the DMA fetches the last k-tile
        // again into a stage that is no longer read.
        barrier_after(std::integral_constant<int, (S - 2) * N_LOAD + (S_B - S) * NBL>{});
        if constexpr (MX) {
#pragma unroll
          for (int q = 0; q < NSC; ++q) s_cur[q] = s_nxt[q];
          if constexpr (SC2) load_scales(s_nxt, min(kt + 2, nk - 1));
        }
        MOE_FENCE();
      }
      int m = 0;  // next memory op
#pragma unroll
      for (int q = H; q < N_MFMA; ++q) {
        // memory ops assigned to the slot before MFMA q
        const int m_end = (q - H + 1) * nm / (N_MFMA - H);
#pragma unroll
        for (int mm = 0; mm < NM_MAX; ++mm) {
          if (mm < m || mm >= m_end) continue;
          // reads spread evenly among the DMAs: op mm is a read iff the
          // running read quota floor(x * N_READ / nm) steps at it
          const int rb = mm * N_READ / nm;
          if ((mm + 1) * N_READ / nm != rb) {
            if constexpr (last)
              read_one(sa_next, sbb_next, 0, nxt, rb);
            else
              read_one(sa, sbb, ks + 1, nxt, rb);
          } else if constexpr (last) {
            issue_one(min(kt + S, nk - 1), st, min(kt + S_B, nk - 1), sbt,
                      d_lo + mm - rb);
          } else {
            issue_one(0, 0, min(kt + S_B - 1, nk - 1), sbt_prev, d_lo + mm - rb);
          }
          MOE_FENCE();
        }
        m = m_end;
        mfma_one(cur, q, sk);
        MOE_FENCE();
      }
    });
    st = st_next;
    st_next = st_next + 1 == S ? 0 : st_next + 1;
    sbt_prev = sbt;
    sbt = sbt_next;
    sbt_next = sbt_next + 1 == S_B ? 0 : sbt_next + 1;
  }
  };
  constexpr bool kTwoCopies = kSkipTail && SKIP == 2 && !(MX && DUAL);
  if (kSkipTail && (!kTwoCopies || act_mb < MB))
    kloop(std::integral_constant<bool, kSkipTail>{});
  else
    kloop(std::false_type{});
#undef MOE_FENCE
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load may still target LDS at exit
  // 16-byte row pieces, through LDS or (TACC) straight from registers: the
  // output (SwiGLU of the two accumulators, or the plain product), then
  // any saved pre-activations. value(i, j, r) is element r of block (i, j);
  // store(row, col, v) takes 8 consecutive columns of one tile row.
  using SO = StageOut<BM, BN, WM, WN, MB, NB, NW * kWave, kEpiRows>;
  auto out = [&](auto value, auto store, int rows) {
    if constexpr (TACC) {
      // quads 2 pr and 2 pr + 1 hold columns 16 pr + 4 half .. +3 and
      // 16 pr + 8 + 4 half .. +3 of row l % 32; after the swap lane l < 32
      // holds 16 pr + 8 .. +15 and lane l + 32 holds 16 pr .. +7
      const int half = lane / 32;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (wm * WM + i * 32 >= rows) continue;  // (wave-uniform)
        const int row = wm * WM + i * 32 + lane % 32;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          float x[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) x[r] = value(i, j, r);
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const auto sw = __builtin_amdgcn_permlane32_swap(
                  __builtin_bit_cast(uint32_t, x[4 * (2 * pr + 1) + e]),
                  __builtin_bit_cast(uint32_t, x[4 * (2 * pr) + e]), false, false);
              x[4 * (2 * pr + 1) + e] = __builtin_bit_cast(float, (uint32_t)sw[0]);
              x[4 * (2 * pr) + e] = __builtin_bit_cast(float, (uint32_t)sw[1]);
            }
            const float v[8] = {x[8 * pr + 4], x[8 * pr + 5], x[8 * pr + 6], x[8 * pr + 7],
                                x[8 * pr], x[8 * pr + 1], x[8 * pr + 2], x[8 * pr + 3]};
            store(row, wn * WN + j * 32 + 16 * pr + (half ? 0 : 8), v);
          }
        }
      }
    } else {
      SO::run(lds, wm, wn, lane, value, store, rows);
    }
  };
  if constexpr (EPI == kEpiSwigluMx) {
    // h through LDS in rows of the tile; each thread then quantises one
    // whole 32-column block of a row: its amax in registers, 32 codes in
    // two 16-byte stores and one scale byte (the accumulator layout spreads
    // a block over a half-wave: a 5-step butterfly per element and one
    // byte store per lane)
    using SO32 = StageOut<BM, BN, WM, WN, MB, NB, NW * kWave, kEpiRows, 32>;
    uint8_t* hq = (uint8_t*)p.C;
    uint8_t* hs = (uint8_t*)p.C2;
    SO32::run(lds, wm, wn, lane,
              [&](int i, int j, int r) {
                const float a = acc[0][i][j][r], b = acc[NB_OPS - 1][i][j][r];
                return a * fast_sigmoid(a) * b;
              },
              [&](int row, int col, const float* v) {
                const int grow = t.m0 + row, gcol = t.n0 + col;
                if (grow >= t.m_end || gcol >= p.N) return;
                float m = 0.0f;
#pragma unroll
                for (int q = 0; q < 32; ++q) m = fmaxf(m, fabsf(v[q]));
                const int X = mx_block_exponent(m);
                const float inv = mx_inv_scale(X);
                uint32_t w[8];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                  w[q] = e4m3_encode(v[4 * q] * inv) |
                         (e4m3_encode(v[4 * q + 1] * inv) << 8) |
                         (e4m3_encode(v[4 * q + 2] * inv) << 16) |
                         (e4m3_encode(v[4 * q + 3] * inv) << 24);
                u32x4* dst = (u32x4*)(hq + (long)grow * p.ldc + gcol);
                dst[0] = u32x4{w[0], w[1], w[2], w[3]};
                dst[1] = u32x4{w[4], w[5], w[6], w[7]};
                hs[mx_scale_index(grow, gcol / 32, p.M)] = (uint8_t)(X + 127);
              },
              t.m_end - t.m0);
    auto put_bf16 = [&](void* dst) {
      return [=](int row, int col, const float* v) {
        const int grow = t.m0 + row, gcol = t.n0 + col;
        if (grow >= t.m_end || gcol >= p.N) return;
        *(bf16x8*)((bf16*)dst + (long)grow * p.ldc + gcol) = pack8(v);
      };
    };
    if (p.Sa)
      SO::run(lds, wm, wn, lane,
              [&](int i, int j, int r) { return acc[0][i][j][r]; },
              put_bf16(p.Sa), t.m_end - t.m0);
    if (p.Sb)
      SO::run(lds, wm, wn, lane,
              [&](int i, int j, int r) { return acc[NB_OPS - 1][i][j][r]; },
              put_bf16(p.Sb), t.m_end - t.m0);
  } else {
    auto put = [&](TO* dst) {
      return [=](int row, int col, const float* v) {
        const int grow = t.m0 + row, gcol = t.n0 + col;
        if (grow >= t.m_end || gcol >= p.N) return;
        TO* o = dst + (long)grow * p.ldc + gcol;
        // a piece that ends past N (N = E of the router, any count), or
        // whose rows are not 16-byte aligned, is stored element by element:
        // its tail columns would land in the next row
        if (gcol + 8 > p.N || (p.ldc * (long)sizeof(TO)) % 16 != 0) {
          const int n = min(8, p.N - gcol);
          for (int q = 0; q < n; ++q) o[q] = from_f32<TO>(v[q]);
          return;
        }
        if constexpr (sizeof(TO) == 2) {
          *(bf16x8*)o = pack8(v);
        } else {
          *(f32x4*)o = f32x4{v[0], v[1], v[2], v[3]};
          *(f32x4*)(o + 4) = f32x4{v[4], v[5], v[6], v[7]};
        }
      };
    };
    if constexpr (EPI == kEpiSwiglu) {
      if (p.C)
        out([&](int i, int j, int r) {
              const float a = acc[0][i][j][r], b = acc[NB_OPS - 1][i][j][r];
              return a * fast_sigmoid(a) * b;
            },
            put((TO*)p.C), t.m_end - t.m0);
      if (p.C2)
        out([&](int i, int j, int r) { return acc[0][i][j][r]; }, put((TO*)p.C2),
            t.m_end - t.m0);
      if (p.C3)
        out([&](int i, int j, int r) { return acc[NB_OPS - 1][i][j][r]; },
            put((TO*)p.C3), t.m_end - t.m0);
    } else if constexpr (EPI == kEpiSwigluBwd) {
      // dh = acc; (da, db) from the pre-activations a, b (bf16, ld = ldc),
      // which may share their buffers with da, db
      out([&](int i, int j, int r) { return acc[0][i][j][r]; },
              [&](int row, int col, const float* v) {
                const int grow = t.m0 + row, gcol = t.n0 + col;
                if (grow >= t.m_end || gcol >= p.N) return;
                const long o = (long)grow * p.ldc + gcol;
                const bf16x8 a8 = *(const bf16x8*)((const bf16*)p.aux_a + o);
                const bf16x8 b8 = *(const bf16x8*)((const bf16*)p.aux_b + o);
                float da[8], db[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                  const float a = (float)a8[q], b = (float)b8[q];
                  const float sg = fast_sigmoid(a);
                  da[q] = v[q] * b * sg * (1.0f + a * (1.0f - sg));
                  db[q] = v[q] * a * sg;
                }
                *(bf16x8*)((bf16*)p.C + o) = pack8(da);
                *(bf16x8*)((bf16*)p.C2 + o) = pack8(db);
              }, t.m_end - t.m0);
    } else {
      out([&](int i, int j, int r) { return acc[0][i][j][r]; },
          put((TO*)p.C + (SCHED == kSchedK ? (long)t.g * p.sC : 0)), t.m_end - t.m0);
    }
  }
}

// Direct-to-LDS form for the backward products (bf16), where operands may
// be stored k-major: element (row r, contraction index k) at base[k*ld + r]
// (the row-major form, base[r*ld + k], is loaded as in the forward). A
// k-major k-tile is DMA'd as it lies: 64 rows of the contraction index,
// each R = BM or BN elements long, its 16-byte chunk c at position
// c ^ (4 * (k & 3)). The MFMA fragment (32 operand rows x 16 k) is read
// with two ds_read_b64_tr_b16: within each 16-lane group, lane j points at
// k-row kb + j/4, elements r0 + 4*(j%4) .. +3, and the transposing read
// hands lane i the four k values kb..kb+3 of element r0 + i. Rows kb..kb+3
// sit in distinct quarters of the 64 banks, so the reads are conflict-free.
//
// SCHED = kSchedK contracts over each group's ragged row range (weight
// gradients: C_g = A_g^T B_g); k-tiles past the range read zeros, since
// every k-tile's buffer resource ends at the range end. (It serves the
// router backward and the weight gradients with outputs below 256 in a
// dimension.)
template <int BM, int BN, int WGM, int WGN, bool A_KM, bool B_KM, int EPI, int SCHED>
__global__ __launch_bounds__(WGM * WGN * kWave) void mfma_gemm_t(GemmParams p) {
  static_assert(EPI == kEpiStore || EPI == kEpiStoreF32 || EPI == kEpiAccum, "epilogue");
  typedef bf16x8 Frag;
  constexpr int NW = WGM * WGN, S = 2;
  constexpr int RB = 128, BK = 64, KS = BK / 16;  // bytes / elements / substeps
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  constexpr int STAGE = A_BYTES + B_BYTES;
  // DMA instructions per wave and k-tile (1 KB each)
  constexpr int A_INS = BM / 8 / NW, B_INS = BN / 8 / NW;
  constexpr int N_LOAD = A_INS + B_INS;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile shape");
  static_assert(BM >= 128 && BN >= 128 && MB >= 1 && NB >= 1, "tile shape");

  constexpr int kEpiRows = BM > 128 ? 128 : BM;
  constexpr int EPI_BYTES = StageOut<BM, BN, WM, WN, MB, NB, NW * kWave, kEpiRows>::BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[S * STAGE > EPI_BYTES ? S * STAGE : EPI_BYTES];

  Tile t;
  if (!lookup_tile<BM, BN, SCHED>(p, t)) return;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WGN, wn = wave % WGN;

  // k-tiles: rows [k_beg, k_end) of the contraction (SCHED K), else [0, K)
  const int kspan = SCHED == kSchedK ? t.k_end - t.k_beg : p.K;
  const int nk = (kspan + BK - 1) / BK;

  // Source of DMA instruction d of operand X (rows [r0, r0 + R) of the
  // tile) for k-tile kt. Row-major: 8 rows of 128 bytes, as the forward.
  // k-major: 1024 / (2R) k-rows of 2R bytes; the resource starts at the
  // k-tile's first row and ends with the valid rows (zeros past them).
  auto dma = [&](const void* X, int ld, int r0, int r_end, int R, bool km,
                 int kt, char* dst, int d) {
    const int kbase = (SCHED == kSchedK ? t.k_beg : 0) + kt * BK;
    if (!km) {
      const int row = (d * NW + wave) * 8 + lane / 8, phys = lane % 8;
      const int grow = min(r0 + row, r_end - 1);
      const Rsrc rs = make_rsrc((const char*)X + (long)r0 * ld * 2);
      dma16(rs, dst, (grow - r0) * ld * 2 + swz<8>(row, phys) * 16, kbase * 2);
    } else {
      const int cpk = R / 8;  // chunks per k-row
      const int kr = (d * NW + wave) * (64 / cpk) + lane / cpk;
      const int c = (lane % cpk) ^ (4 * (kr & 3));
      const int rows_left = SCHED == kSchedK ? t.k_end - kbase : kspan - kt * BK;
      const char* base = (const char*)X + ((long)kbase * ld + r0) * 2;
      dma16(make_rsrc_n(base, ((long)rows_left * ld - r0) * 2), dst,
            kr * ld * 2 + c * 16, 0);
    }
  };
  const void* Bop = (const char*)p.B + (SCHED == kSchedM ? (long)t.g * p.sB * 2 : 0);
  auto issue_one = [&](int kt, int stage, int d) {
    char* base = lds + stage * STAGE;
    if (d < A_INS) {
      dma(p.A, p.lda, t.m0, t.m_end, BM, A_KM, kt, base + (d * NW + wave) * 1024, d);
    } else {
      const int j = d - A_INS;
      dma(Bop, p.ldb, t.n0, p.N, BN, B_KM, kt, base + A_BYTES + (j * NW + wave) * 1024, j);
    }
  };
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int d = 0; d < N_LOAD; ++d) issue_one(kt, stage, d);
  };

  // fragment reads: row-major as in the forward; k-major by two transposing
  // reads of 4 k each
  const int lrow = lane % 32, half = lane / 32, sw = (lrow >> 1) & 7;
  const int grp = lane / 16, gj = lane % 16;
  auto read_rm = [&](const char* op, int row0, int ks) {
    return *(const Frag*)(op + (row0 + lrow) * RB + (((ks * 2 + half) ^ sw) * 16));
  };
  auto read_km = [&](const char* op, int R, int row0, int ks) {
    const int r = row0 + 16 * (grp & 1) + 4 * (gj & 3);
    s16x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = ks * 16 + 8 * (grp >> 1) + 4 * h + (gj >> 2);
      const int c = (r >> 3) ^ (4 * (k & 3));
      v[h] = lds_read_tr16(op + k * (R * 2) + c * 16 + (r & 7) * 2);
    }
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 w = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(Frag, w);
  };
  struct Frags {
    Frag a[MB], b[NB];
  };
  constexpr int N_READ = MB + NB;
  constexpr int N_MFMA = MB * NB;
  // reads in the order the substep's MFMAs first use the fragments, on
  // the big tiles (measured: the 2 x 2 block tiles run faster A then B)
  constexpr ReadOrder<MB, NB, 1, (N_MFMA >= 8)> kOrder{};
  auto read_one = [&](const char* sb, int ks, Frags& f, int m) {
    const int r = kOrder.r[m];
    if (r < MB) {
      const int row0 = wm * WM + r * 32;
      f.a[r] = A_KM ? read_km(sb, BM, row0, ks) : read_rm(sb, row0, ks);
    } else {
      const int j = r - MB, row0 = wn * WN + j * 32;
      f.b[j] = B_KM ? read_km(sb + A_BYTES, BN, row0, ks)
                    : read_rm(sb + A_BYTES, row0, ks);
    }
  };

  f32x16 acc[1][MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[0][i][j] = f32x16{};
  auto mfma_one = [&](const Frags& f, int q) {
    const int i = q / NB, j = q % NB;
    acc[0][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j],
                                                           acc[0][i][j], 0, 0, 0);
  };
  auto barrier_after = [&](auto vm_left) {
    tile_barrier<decltype(vm_left)::value>();
  };

  if (nk > 0) {
    issue(0, 0);
    issue(min(1, nk - 1), 1);
    barrier_after(std::integral_constant<int, N_LOAD>{});
    Frags fa, fb;
#pragma unroll
    for (int r = 0; r < N_READ; ++r) read_one(lds, 0, fa, r);
    // the forward kernel's fenced schedule: each substep's MFMAs with the
    // next substep's reads (and, at the last, the DMA of tile kt+2) spread
    // among them; branch-free at the end so the wait counts stay exact
    constexpr int H = N_MFMA >= 8 ? 2 : 1;
#define MOE_FENCE() __builtin_amdgcn_sched_barrier(0)
    for (int kt = 0; kt < nk; ++kt) {
      const char* sb = lds + (kt & 1) * STAGE;
      const char* sb_next = lds + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        Frags& cur = (ks & 1) ? fb : fa;
        Frags& nxt = (ks & 1) ? fa : fb;
        const bool last = ks + 1 == KS;
        constexpr int NM_MAX = N_READ + N_LOAD;
        const int nm = last ? NM_MAX : N_READ;
        MOE_FENCE();
#pragma unroll
        for (int q = 0; q < H; ++q) mfma_one(cur, q);
        MOE_FENCE();
        if (last) {
          barrier_after(std::integral_constant<int, 0>{});
          MOE_FENCE();
        }
        int m = 0;
#pragma unroll
        for (int q = H; q < N_MFMA; ++q) {
          const int m_end = (q - H + 1) * nm / (N_MFMA - H);
#pragma unroll
          for (int mm = 0; mm < NM_MAX; ++mm) {
            if (mm < m || mm >= m_end) continue;
            if (!last) {
              read_one(sb, ks + 1, nxt, mm);
            } else {
              const int rb = mm * N_READ / NM_MAX;
              if ((mm + 1) * N_READ / NM_MAX != rb)
                read_one(sb_next, 0, nxt, rb);
              else
                issue_one(min(kt + 2, nk - 1), kt & 1, mm - rb);
            }
            MOE_FENCE();
          }
          m = m_end;
          mfma_one(cur, q);
          MOE_FENCE();
        }
      }
    }
#undef MOE_FENCE
    __builtin_amdgcn_s_waitcnt(0);  // no load may still target LDS at exit
  }
  // through LDS: ROWS rows per pass (the stages are free now)
  const long c_off = SCHED == kSchedK ? (long)t.g * p.sC : 0;
  bf16* C = (bf16*)p.C + c_off;
  auto value = [&](int i, int j, int r) { return acc[0][i][j][r]; };
  auto store = [&](int row, int col, const float* v) {
    const int grow = t.m0 + row, gcol = t.n0 + col;
    if (grow >= t.m_end || gcol >= p.N) return;
    const long o = (long)grow * p.ldc + gcol;
    if constexpr (EPI == kEpiStore) {
      *(bf16x8*)(C + o) = pack8(v);
    } else if constexpr (EPI == kEpiStoreF32) {
      float* Cf = (float*)p.C + c_off + o;
      *(f32x4*)Cf = f32x4{v[0], v[1], v[2], v[3]};
      *(f32x4*)(Cf + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {  // kEpiAccum
      const bf16x8 c8 = *(const bf16x8*)(C + o);
      float s[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] = (float)c8[q] + v[q];
      *(bf16x8*)(C + o) = pack8(s);
    }
  };
  StageOut<BM, BN, WM, WN, MB, NB, NW * kWave, kEpiRows>::run(lds, wm, wn, lane,
                                                              value, store, t.m_end - t.m0);
}

// Weight gradients C_g = A_g^T B_g over each group's row range (the
// contraction-grouped products, both operands k-major: element (r, k) at
// X[k * ld + r]) as a persistent kernel. Workgroup b takes the tiles
// first + j * gridDim.x (first: b's slot, each XCD a contiguous share of
// every round of tiles) and runs them as one stream of k-tiles: during the
// k-tile of step s it issues the DMA of step s + 2, also when that step
// belongs to its next tile, so a tile's first operands arrive while the
// tile before it still computes. An empty row range is one k-tile of zeros
// (the tile stores zeros). The MFMAs take their operands swapped and
// accumulate C^T: element r of lane l is C row l % 32, column
// 8 (r / 4) + 4 (l / 32) + r % 4 of the 32 x 32 block, so a register quad
// holds four consecutive columns of one row. A swap of lane halves
// (v_permlane32_swap) gathers eight, and the epilogue stores 16-byte row
// pieces straight from registers, with no LDS staging and no barrier,
// while the next tile's DMA is in flight.
//
// RING: as in the forward kernel, B runs in a ring of three stages and A
// in two (all 160 KB of LDS): the B DMA of step s + 2 goes into the B stage
// of step s - 1 and is spread over substeps 0 .. KS-2 of step s, and only
// A's DMA follows the tile barrier, whose wait then leaves those B loads
// in flight. After a tile's stores the barrier waits for everything
// (loads and stores retire out of order with each other).
template <int BM, int BN, int WGM, int WGN, bool RING = true, int DW = WGM * WGN>
__global__ __launch_bounds__(WGM * WGN * kWave) void mfma_wgrad(GemmParams p) {
  typedef bf16x8 Frag;
  constexpr int NW = WGM * WGN;
  constexpr int RB = 128, BK = 64, KS = BK / 16;  // bytes / elements / substeps
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB;
  constexpr int SB = RING ? 3 : 2;  // B stages (A: 2)
  constexpr int B_BASE = 2 * A_BYTES;
  // DMA instructions per wave and k-tile (1 KB each)
  constexpr int A_INS = BM / 8 / NW, B_INS = BN / 8 / NW;
  constexpr int N_LOAD = A_INS + B_INS, NBL = B_INS;
  static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile shape");
  static_assert(BM >= 128 && BN >= 128 && BM <= 512 && BN <= 512, "tile shape");
  static_assert(2 * A_BYTES + SB * B_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) char lds[2 * A_BYTES + SB * B_BYTES];

  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WGN, wn = wave % WGN;
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles_mn = (p.M + BM - 1) / BM * tiles_n;
  const int n_tiles = p.G * tiles_mn;
  const int grid = (int)gridDim.x;
  const int first = xcd_remap_n((int)blockIdx.x, grid);
  const int km = p.kmul > 0 ? p.kmul : 1;
  // the group offsets through the constant address space: scalar loads,
  // whose wait (lgkmcnt) leaves the DMA and stores in flight (a vector
  // load here would wait for all of them)
  typedef const __attribute__((address_space(4))) int32_t* OffPtr;
  const OffPtr off = (OffPtr)p.off;

  // a position in the k-tile stream: tile j of this workgroup, its k-tile kt
  struct Cur {
    int j, kt, nk, g, m0, n0, k_beg, k_end;
  };
  auto start_tile = [&](Cur& c) {  // first k-tile of tile c.j; false past the end
    const int L = first + c.j * grid;
    if (L >= n_tiles) return false;
    c.g = L / tiles_mn;
    const int rem = L - c.g * tiles_mn;
    c.m0 = rem / tiles_n * BM;
    c.n0 = rem % tiles_n * BN;
    c.k_beg = off[c.g] * km;
    c.k_end = off[c.g + 1] * km;
    c.nk = max(1, (c.k_end - c.k_beg + BK - 1) / BK);
    c.kt = 0;
    return true;
  };
  auto next_step = [&](Cur& c) {
    if (++c.kt < c.nk) return true;
    ++c.j;
    return start_tile(c);
  };

  // DMA instruction d of the k-tile at c into stage st (d < A_INS: A's
  // rows [m0, m0 + BM), else B's [n0, n0 + BN)), as it lies: 1024 / (2R)
  // k-rows of R elements, 16-byte chunk ch of k-row k at position
  // ch ^ (4 (k & 3)). The resource ends with the group's rows, so k-rows
  // past them read zeros; live = false (past the last step) reads zeros
  // only.
  static_assert(NW % DW == 0 && DW >= 1, "DMA waves");
  auto issue_one = [&](const Cur& c, bool live, int sa, int sb, bool is_a, int jd) {
    const int cpk = (is_a ? BM : BN) / 8;  // chunks per k-row
    const int kr = (jd * DW + wave) * (64 / cpk) + lane / cpk;
    const int ch = (lane % cpk) ^ (4 * (kr & 3));
    const int kbase = c.k_beg + c.kt * BK;
    const int rows_left = live ? c.k_end - kbase : 0;
    const long ld = is_a ? p.lda : p.ldb;
    const int r0 = is_a ? c.m0 : c.n0;
    const char* base = (const char*)(is_a ? p.A : p.B) + ((long)kbase * ld + r0) * 2;
    char* dst = (is_a ? lds + sa * A_BYTES : lds + B_BASE + sb * B_BYTES) +
                (jd * DW + wave) * 1024;
    dma16(make_rsrc_n(base, ((long)rows_left * ld - r0) * 2), dst,
          kr * (int)ld * 2 + ch * 16, 0);
  };

  // fragment (32 rows x 16 k) by two transposing reads of 4 k each: within
  // each 16-lane group lane j points at k-row kb + j / 4, elements
  // r0 + 4 (j % 4) .. +3, and lane i receives the four k of element r0 + i
  const int grp = lane / 16, gj = lane % 16;
  auto read_km = [&](const char* op, int R, int row0, int ks) {
    const int r = row0 + 16 * (grp & 1) + 4 * (gj & 3);
    s16x4 v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = ks * 16 + 8 * (grp >> 1) + 4 * h + (gj >> 2);
      const int c = (r >> 3) ^ (4 * (k & 3));
      v[h] = lds_read_tr16(op + k * (R * 2) + c * 16 + (r & 7) * 2);
    }
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 w = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(Frag, w);
  };
  struct Frags {
    Frag a[MB], b[NB];
  };
  constexpr int N_READ = MB + NB;
  constexpr int N_MFMA = MB * NB;
  constexpr ReadOrder<MB, NB, 1, (N_MFMA >= 8)> kOrder{};
  auto read_one = [&](const char* pa, const char* pb, int ks, Frags& f, int m) {
    const int r = kOrder.r[m];
    if (r < MB)
      f.a[r] = read_km(pa, BM, wm * WM + r * 32, ks);
    else
      f.b[r - MB] = read_km(pb, BN, wn * WN + (r - MB) * 32, ks);
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};
  auto mfma_one = [&](const Frags& f, int q) {  // C^T block (i, j)
    const int i = q / NB, j = q % NB;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };

  // the finished tile at c from registers: block (i, j), quads 2 pr and
  // 2 pr + 1 packed to bf16 (columns 16 pr + 4 half .. and 16 pr + 8 +
  // 4 half ..), lane halves swapped so that lane l < 32 holds columns
  // 16 pr + 8 .. +15 and lane l + 32 columns 16 pr .. +7 of row l
  // (inlined: a call would keep acc in scratch memory)
  auto store_tile = [&](const Cur& c) __attribute__((always_inline)) {
    constexpr bool BFLY = NB == 2 && DW == NW;
    bf16* C = (bf16*)p.C + (long)c.g * p.sC;
    const int half = lane / 32;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      u32x4 vj[2][2];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        uint32_t w[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const bf16 lo = (bf16)acc[i][j][4 * q + 2 * h];
            const bf16 hi = (bf16)acc[i][j][4 * q + 2 * h + 1];
            w[q][h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
        u32x4 v[2];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const auto sw = __builtin_amdgcn_permlane32_swap(w[2 * pr + 1][h], w[2 * pr][h],
                                                             false, false);
            w[2 * pr + 1][h] = sw[0];
            w[2 * pr][h] = sw[1];
          }
          // columns 16 pr + 8 .. +15 of row lane % 32 (lanes 0-31), 16 pr ..
          // +7 (lanes 32-63)
          v[pr] = u32x4{w[2 * pr + 1][0], w[2 * pr + 1][1], w[2 * pr][0], w[2 * pr][1]};
        }
        // Swap the odd 16-lane rows of v[0] with the even ones of v[1]: v[0]
        // then holds rows 0-15 of the block, v[1] rows 16-31, with lanes o,
        // 16 + o, 32 + o, 48 + o holding columns 8, 24, 0, 16 (+0 .. 7) of
        // row o. Each store then writes 16 rows x 64 bytes, not 32 x 32.
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto sw = __builtin_amdgcn_permlane16_swap(v[0][e], v[1][e], false, false);
          v[0][e] = sw[0];
          v[1][e] = sw[1];
        }
        if constexpr (!BFLY) {
          const int col = c.n0 + wn * WN + j * 32 + 16 * ((lane >> 4) & 1) + (half ? 0 : 8);
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const int row = c.m0 + wm * WM + i * 32 + 16 * pr + lane % 16;
            if (row < p.M && col < p.N) *(u32x4*)(C + (long)row * p.ldc + col) = v[pr];
          }
        } else {
          vj[j][0] = v[0];
          vj[j][1] = v[1];
        }
        acc[i][j] = f32x16{};
      }
      if constexpr (BFLY) {
        // exchange the column half (j) with lane bit 3 (rows o and o ^ 8 of
        // a 16-lane row): register k then holds rows 16 pr + 8 k + lane % 8,
        // all 64 columns (lane bit 3 the half), 8 rows x 128 bytes a store.
        // Only where every wave waits for its stores at the next barrier
        // (all waves issue DMA): there whole lines drain faster (DeepSeek-V3
        // dW1 + dW3 5.12 -> 4.86 ms); with half of the waves loading, the
        // extra exchange costs more than it saves (Mixtral, skewed and
        // Qwen-MoE-like weight gradients 2-4% slower).
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          const bool up = (lane & 8) != 0;
          u32x4 n0, n1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x1 = (uint32_t)__builtin_amdgcn_update_dpp(
                0, (int)vj[1][pr][e], 0x128, 0xf, 0xf, false);  // row_ror:8
            const uint32_t x0 = (uint32_t)__builtin_amdgcn_update_dpp(
                0, (int)vj[0][pr][e], 0x128, 0xf, 0xf, false);
            n0[e] = up ? x1 : vj[0][pr][e];
            n1[e] = up ? vj[1][pr][e] : x0;
          }
          const int col = c.n0 + wn * WN + 32 * ((lane >> 3) & 1) + 16 * ((lane >> 4) & 1) +
                          (half ? 0 : 8);
          const int row0 = c.m0 + wm * WM + i * 32 + 16 * pr + (lane & 7);
          if (row0 < p.M && col < p.N) *(u32x4*)(C + (long)row0 * p.ldc + col) = n0;
          if (row0 + 8 < p.M && col < p.N) *(u32x4*)(C + (long)(row0 + 8) * p.ldc + col) = n1;
        }
      }
    }
  };

  Cur cc;
  cc.j = 0;
  if (!start_tile(cc)) return;

  // DW < NW: only waves 0 .. DW-1 issue the DMA (NW / DW times their share
  // each). The others never wait for the vector-memory counter, so their
  // tile barrier waits for no stores of theirs; the barrier still releases
  // only once the DMA waves have their loads (and their own stores) done.
  auto run = [&](auto role) {
    constexpr bool DMAW = decltype(role)::value;
    constexpr int AI = DMAW ? A_INS * NW / DW : 0;  // A / B DMA per wave and step
    constexpr int BI = DMAW ? B_INS * NW / DW : 0;
    constexpr int NL = AI + BI;
    auto issue = [&](const Cur& c, bool live, int sa_, int sb_, int d) {
      if constexpr (DMAW) issue_one(c, live, sa_, sb_, d < AI, d < AI ? d : d - AI);
    };
    auto barrier_n = [&](auto n) {  // wait for this wave's DMA, leaving n
      if constexpr (DMAW) tile_barrier<decltype(n)::value>();
      else tile_barrier<63>();  // (LDS reads only)
    };
    // prologue: steps 0 and 1 into stages 0 and 1, the load cursor at step 2
    Cur cl = cc;
#pragma unroll
    for (int d = 0; d < NL; ++d) issue(cl, true, 0, 0, d);
    bool live = next_step(cl);
#pragma unroll
    for (int d = 0; d < NL; ++d) issue(cl, live, 1, 1, d);
    live = live && next_step(cl);
    barrier_n(std::integral_constant<int, NL>{});
    Frags fa, fb;
#pragma unroll
    for (int r = 0; r < N_READ; ++r) read_one(lds, lds + B_BASE, 0, fa, r);

    // One region per k-substep, as the backward kernel's: the substep's
    // MFMAs with the next substep's fragment reads (and the DMA of step
    // s + 2) spread among them.
    constexpr int H = N_MFMA >= 8 ? 2 : 1;
#define MOE_FENCE() __builtin_amdgcn_sched_barrier(0)
    int sa = 0;                                   // A stage of step s
    int sbt = 0, sbt_next = 1, sbt_prev = SB - 1;  // B stages of steps s, s+1, s-1
    bool stores_out = false;  // a tile's stores issued since the last full wait
    for (;;) {
      const char* pa = lds + sa * A_BYTES;
      const char* pa_next = lds + (sa ^ 1) * A_BYTES;
      const char* pb = lds + B_BASE + sbt * B_BYTES;
      const char* pb_next = lds + B_BASE + sbt_next * B_BYTES;
      static_for<KS>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        Frags& cur = (ks & 1) ? fb : fa;
        Frags& nxt = (ks & 1) ? fa : fb;
        constexpr bool last = ks + 1 == KS;
        // memory ops of this region: N_READ reads and the DMA instructions
        // [d_lo, d_hi) of step s + 2 (with the ring: A's after the
        // barrier, a share of B's at each earlier substep; else all after)
        constexpr int NM_MAX = N_READ + NL;
        constexpr int d_lo = !RING || last ? 0 : AI + ks * BI / (KS - 1);
        constexpr int d_hi = !RING ? (last ? NL : 0)
                             : last ? AI
                                    : AI + (ks + 1) * BI / (KS - 1);
        constexpr int nm = N_READ + d_hi - d_lo;
        MOE_FENCE();
#pragma unroll
        for (int q = 0; q < H; ++q) mfma_one(cur, q);
        MOE_FENCE();
        if constexpr (last) {
          // the DMA of step s + 1 (with the ring, B's of step s + 2 may stay
          // in flight); after a tile's stores everything
          if (!RING || stores_out) {
            barrier_n(std::integral_constant<int, 0>{});
            stores_out = false;
          } else {
            barrier_n(std::integral_constant<int, BI>{});
          }
          MOE_FENCE();
        }
        int m = 0;
#pragma unroll
        for (int q = H; q < N_MFMA; ++q) {
          const int m_end = (q - H + 1) * nm / (N_MFMA - H);
#pragma unroll
          for (int mm = 0; mm < NM_MAX; ++mm) {
            if (mm < m || mm >= m_end) continue;
            const int rb = mm * N_READ / nm;
            if ((mm + 1) * N_READ / nm != rb) {
              if constexpr (last)
                read_one(pa_next, pb_next, 0, nxt, rb);
              else
                read_one(pa, pb, ks + 1, nxt, rb);
            } else {
              issue(cl, live, sa, RING ? sbt_prev : sbt, d_lo + mm - rb);
            }
            MOE_FENCE();
          }
          m = m_end;
          mfma_one(cur, q);
          MOE_FENCE();
        }
      });
      if (cc.kt + 1 == cc.nk) {
        store_tile(cc);
        stores_out = true;
        ++cc.j;
        if (!start_tile(cc)) break;
      } else {
        ++cc.kt;
      }
      if (live) live = next_step(cl);
      sa ^= 1;
      sbt_prev = sbt;
      sbt = sbt_next;
      sbt_next = sbt_next + 1 == SB ? 0 : sbt_next + 1;
    }
#undef MOE_FENCE
  };
  if (DW == NW || wave < DW)
    run(std::true_type{});
  else
    run(std::false_type{});
  __builtin_amdgcn_s_waitcnt(0);  // no load may still target LDS at exit
}

template <int BM, int BN, int WGM, int WGN, bool A_KM, bool B_KM, int EPI, int SCHED>
hipError_t launch_t(const GemmParams& p, hipStream_t s) {
  const long tiles = launch_grid<BM, BN, SCHED>(p);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mfma_gemm_t<BM, BN, WGM, WGN, A_KM, B_KM, EPI, SCHED>),
                     dim3((unsigned)tiles), dim3(WGM * WGN * kWave), 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN, bool A_KC, bool B_KC,
          bool DUAL, int EPI, int SCHED, typename TO>
hipError_t launch(const GemmParams& p, hipStream_t s) {
  const long tiles = launch_grid<BM, BN, SCHED>(p);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(
      (mfma_gemm<BM, BN, BK, WGM, WGN, A_KC, B_KC, DUAL, EPI, SCHED, TO>),
      dim3((unsigned)tiles), dim3(WGM * WGN * kWave), 0, s, p);
  return hipGetLastError();
}

template <int BM, int BN, int S, int WGM, int WGN, bool DUAL, int EPI,
          typename TO, bool MX, int SCHED = kSchedM, int TAIL = 0,
          int SKIP = 0, bool KCAT = false, int SB = 0, bool BKM = false>
hipError_t launch_dl(const GemmParams& p, hipStream_t s) {
  const long tiles = launch_grid<BM, BN, SCHED, TAIL>(p);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((mfma_gemm_dl<BM, BN, S, WGM, WGN, DUAL, EPI, TO, MX, SCHED, TAIL, SKIP, KCAT, SB, BKM>),
                     dim3((unsigned)tiles), dim3(WGM * WGN * kWave), 0, s, p);
  return hipGetLastError();
}

// waves of a big direct-to-LDS tile: 4 or 8 (MOE_BIG_TILE_WAVES, for tuning)
// waves of a big direct-to-LDS tile forced by MOE_BIG_TILE_WAVES (4 or 8,
// for tuning), else 0
int big_tile_waves() {
  static const int v = [] {
    const char* e = tuning_env("MOE_BIG_TILE_WAVES");
    const int n = e ? atoi(e) : 0;
    return n == 4 || n == 8 ? n : 0;
  }();
  return v;
}


// compute units of the current device (cached per device)
int num_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
            hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// the persistent weight-gradient kernel: one workgroup per CU (fewer when
// there are fewer tiles)
template <int BM, int BN, int WGM, int WGN, bool RING = true, int DW = WGM * WGN>
hipError_t launch_wgrad(const GemmParams& p, hipStream_t s) {
  const long tiles = (long)p.G * ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7fffffffL) return hipErrorInvalidValue;
  const long grid = tiles < num_cus() ? tiles : num_cus();
  hipLaunchKernelGGL((mfma_wgrad<BM, BN, WGM, WGN, RING, DW>), dim3((unsigned)grid),
                     dim3(WGM * WGN * kWave), 0, s, p);
  return hipGetLastError();
}

template <bool DUAL, int EPI, typename TO, bool MX = false, int SKIP = 0>
hipError_t launch_dl_sized(bool big, const GemmParams& p, hipStream_t s) {
  // big: 256 x 256 outputs (256 x 128 x 2 dual), either over 8 waves, two
  // per SIMD, each holding 128 x 64 (128 x 32 x 2) in accumulators, or over
  // 4 waves, one per SIMD, each holding 128 x 128 (128 x 64 x 2). Eight
  // waves hide latency better and win (the single-B MXFP8 product too,
  // since its scale words take one 32-bit offset per block: MXFP8 GEMM 2
  // 0.915 -> 0.88 ms and the MX dgrad2 1.86 -> 1.57 ms on the Mixtral
  // shape); the 4-wave single-B forms remain for comparison
  // (MOE_BIG_TILE_WAVES=4), and the dual products' 4-wave forms, which
  // spill, are not built.
  if (big) {
    const int forced = big_tile_waves();
    constexpr bool can4 = !DUAL;
    if (can4 && forced == 4) {
      if constexpr (can4)
        return launch_dl<256, DUAL ? 128 : 256, 2, 2, 2, DUAL, EPI, TO, MX>(p, s);
    }
    // Row-grouped products (all but the dual MXFP8 one): a partial last
    // round of big tiles runs as quarter tiles (128 x 128, or 128 x 64 x 2
    // dual) in a second launch.
    // B runs in a 3-stage ring of its own (A in 2, all 160 KB of LDS), so
    // two k-tiles of weights are in flight. Groups of about half a tile
    // (SKIP) stream their weights with too little MFMA work per k-tile to
    // cover one k-tile of HBM latency (measured on the DeepSeek-V3 shape:
    // GEMM 1 3.37 -> 3.12 ms); the full tiles gain less (Mixtral-shaped
    // GEMM 2 1.75 -> 1.69 ms, GEMM 1 3.38 -> 3.36 ms; MXFP8 GEMM 2
    // 1.24 -> 1.18 ms, measured on its 4-wave tile)
    constexpr int SB = 3;
    if constexpr (!MX || !DUAL) {  // (the dual MXFP8 product gained nothing)
      if (p.slots != 0 && p.off) {
        GemmParams q = p;
        if (q.slots < 0) q.slots = num_cus();
        hipError_t e = launch_dl<256, DUAL ? 128 : 256, 2, 2, 4, DUAL, EPI, TO,
                                 MX, kSchedM, 1, SKIP, false, SB>(q, s);
        if (e != hipSuccess) return e;
        return launch_dl<128, DUAL ? 64 : 128, 2, 2, 2, DUAL, EPI, TO, MX,
                         kSchedM, 2, SKIP>(q, s);
      }
    }
    return launch_dl<256, DUAL ? 128 : 256, 2, 2, 4, DUAL, EPI, TO, MX, kSchedM,
                     0, SKIP, false, SB>(p, s);
  }
  return launch_dl<128, DUAL ? 64 : 128, 2, 2, 2, DUAL, EPI, TO, MX>(p, s);
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

// MOE_GEMM_BACKEND=staged keeps the register-staged kernel for every
// product (a testing aid: both kernels must agree with the oracle).
bool force_staged() {
  static const bool v = [] {
    const char* e = tuning_env("MOE_GEMM_BACKEND");
    return e && strcmp(e, "staged") == 0;
  }();
  return v;
}

// n-tiles per rasterization group for a product of tiles_n column tiles:
// all of them when there are at most 8 (the row tiles of an expert then
// run back to back over its whole weight panel: skewed shape, GEMM 1
// 0.898 -> 0.867 ms), else 4 (Mixtral and DeepSeek-V3 shapes, where wider
// groups measured slower). MOE_TILE_GROUP_N overrides, for tuning.
int tile_group_n(int tiles_n) {
  static const int v = [] {
    const char* e = tuning_env("MOE_TILE_GROUP_N");
    const int n = e ? atoi(e) : 0;
    return n > 0 ? n : 0;
  }();
  if (v > 0) return v;
  return tiles_n <= 8 ? (tiles_n > 0 ? tiles_n : 1) : 4;
}

bool mfma_supported(GemmOp op, const GemmParams& p) {
  // 16-byte chunk loads need K (and K1) in multiples of 8; the k-tile of
  // a K-concatenation must not straddle the seam; transposed (row
  // contiguous) operands are loaded 8 rows at a time.
  if (p.K % 8) return false;
  // MXFP8 products run only on the direct-to-LDS kernel: whole 128-byte
  // k-tiles (K % 128) and 32-column scale blocks in the output (N % 32);
  // the scale arrays' byte offsets (rows x K / 32) fit the 32-bit buffer
  // offsets
  if ((op == kOpGemm1Mx || op == kOpGemm2Mx || op == kOpGemm1MxAct ||
       op == kOpDgrad2Mx) &&
      (p.K % 128 || p.N % 32 || p.s_rows * (p.K / 32) > INT_MAX ||
       (long)(p.off ? p.G : 1) * p.N * (p.K / 32) > INT_MAX))
    return false;
  if (op == kOpDgrad1 && p.K1 % 64) return false;
  if ((op == kOpDgrad2 || op == kOpDgrad1) && p.N % 8) return false;
  if (op == kOpWgrad && (p.M % 8 || p.N % 8)) return false;
  // router backward: d_logits rows padded to whole k-tiles (row-major A
  // of the dx product), 16-byte aligned k-rows and output pieces
  if (op == kOpRouterDx && (p.lda % 64 || p.ldb % 8 || p.N % 8)) return false;
  if (op == kOpRouterDw && (p.lda % 8 || p.ldb % 8 || p.N % 8)) return false;
  return true;
}

// MOE_WGRAD_PERSIST=0 keeps the weight gradients on the tile-per-workgroup
// backward kernel, 2 runs the persistent one without its B ring, 3 and 4
// with the DMA from half of the waves or from all of them whatever the
// group sizes, for comparison
int wgrad_persist() {
  static const int v = [] {
    const char* e = tuning_env("MOE_WGRAD_PERSIST");
    return e ? atoi(e) : 1;
  }();
  return v;
}

bool gemm1_gather_supported(int K) { return K % 64 == 0 && !force_staged(); }

bool gemm_direct_ok() { return !force_staged(); }

hipError_t gemm_mfma(GemmOp op, GemmParams p,
                     const int32_t* const* tile_off_by_bm, hipStream_t s) {
  if (!mfma_supported(op, p)) return hipErrorNotSupported;
  // gathered rows only on the direct-to-LDS GEMM 1
  if (p.gsrc && !(op == kOpGemm1Mx ||
                  (op == kOpGemm1 && gemm1_gather_supported(p.K))))
    return hipErrorNotSupported;
  // Big tiles when the average group has enough rows to fill them.
  // skip: one 256-row tile per group with the empty 32-row blocks' MFMAs
  // skipped; tskip: the same skip in big tiles of groups below 1024 rows
  bool big, skip = false, tskip = false;
  if (op == kOpWgrad || op == kOpRouterDw) {
    big = p.M >= 256 && p.N >= 256;
  } else if (op == kOpRouterDx) {
    big = false;
    p.tiles_m_max = (p.M + 127) / 128;
  } else {
    const long rows_per_group = p.off ? (long)p.M / (p.G > 0 ? p.G : 1) : p.M;
    big = rows_per_group >= 192 && p.N >= 256;
    if (op == kOpRouter) big = false;
    // bf16 forward GEMMs whose groups average 96-191 rows: one 256-row
    // tile per group, most groups' weights streamed once, the empty
    // 32-row blocks' MFMAs skipped (DeepSeek-V3 shape, ~128 rows per
    // expert: GEMM 1 3.78 -> 3.37 ms, GEMM 2 2.39 -> 2.22 ms; 128-row
    // tiles give ~half the experts a second, nearly empty tile, and
    // 64-row tiles measured slower still)
    if (!big && p.off && rows_per_group >= 96 && p.N >= 256 &&
        (op == kOpGemm1 || op == kOpGemm2 || op == kOpDgrad2 || op == kOpDgrad1 ||
         op == kOpGemm1Mx || op == kOpGemm1MxAct))
      big = skip = true;
    // bf16 forward products with big groups: each group's ragged last
    // tile skips its empty blocks' MFMAs too, while the waves of full
    // tiles run the copy of the k-loop without the skip branches (Mixtral
    // shape: GEMM 1 3.09 -> 3.02 ms; skewed forward 754 -> 777 TFLOP/s;
    // Qwen-MoE-like layer, ~546 rows per expert: GEMM 1 0.47 -> 0.44 ms).
    // The dual MXFP8 tile has one copy, whose per-MFMA branches cost full
    // tiles about 2%, so there only groups under 4 big tiles take it.
    if (big && !skip && p.off &&
        (op == kOpGemm1 || op == kOpGemm2 ||
         (op == kOpGemm1Mx && rows_per_group < 1024)))
      tskip = true;
    const int bm = op == kOpRouter ? 32 : big ? 256 : 128;
    if (p.off) {
      p.tile_off = tile_off_by_bm[tile_bm_slot(bm)];
      p.tiles_m_max = (p.M + bm - 1) / bm + (p.G < p.M ? p.G : p.M);
    } else {
      p.tiles_m_max = (p.M + bm - 1) / bm;
    }
  }
  {  // column tile width of the kernel chosen below; the backward
     // products keep groups of 4 (wider ones measured slower for dgrad1)
    const bool dual = op == kOpGemm1 || op == kOpGemm1Mx || op == kOpGemm1MxAct;
    const bool fwd = dual || op == kOpGemm2 || op == kOpGemm2Mx || op == kOpRouter;
    const int bn = op == kOpRouter ? 32
                   : dual ? (big ? 128 : 64) : (big ? 256 : 128);
    p.group_n = tile_group_n(fwd ? (p.N + bn - 1) / bn : 1 << 30);
    // one row tile per group (skip): nothing re-reads B, while every
    // column tile of a group reads the same A rows, so all of a group's
    // column tiles run side by side and A leaves HBM once
    // (measured on the DeepSeek-V3 shape: GEMM 2 2.15 -> 2.04 ms, the
    // backward dgrad1 4.95 -> 4.85 ms)
    if (skip) {
      const int bns = fwd ? bn : 256;  // the backward's skip tiles: 256 x 256
      p.group_n = (p.N + bns - 1) / bns;
    }
  }
  // k-contiguous operands with whole k-tiles go straight to LDS
  if (p.K % 64 == 0 && !force_staged()) {
    switch (op) {
      case kOpRouter:
        // Up to 32 experts, one contraction: one wave per 32 x 32 tile,
        // eight k-tiles in flight, so the skinny product spreads over
        // every CU and hides latency. Otherwise a contraction-grouped
        // launch with arithmetic ranges: p.G splits of p.kmul columns of
        // d_model (the partial products at C + g * sC, summed by the
        // top-K kernel), on tiles as wide as the experts allow (64 x 256
        // above 64 experts), so x leaves HBM once and every column tile
        // streams only its split of W_r.
        if (p.G > 1 || p.N > 32) {
          if (p.off || p.kmul % 64 || p.kmul <= 0) return hipErrorInvalidValue;
          if (p.N <= 32)
            return launch_dl<32, 32, 8, 1, 1, false, kEpiStore, float, false,
                             kSchedK>(p, s);
          if (p.N <= 64)
            return launch_dl<64, 64, 4, 2, 2, false, kEpiStore, float, false,
                             kSchedK>(p, s);
          return launch_dl<64, 256, 4, 2, 2, false, kEpiStore, float, false,
                           kSchedK>(p, s);
        }
        return launch_dl<32, 32, 8, 1, 1, false, kEpiStore, float, false>(p, s);
      case kOpGemm1:
        if (skip) return launch_dl_sized<true, kEpiSwiglu, bf16, false, 1>(big, p, s);
        if (tskip) return launch_dl_sized<true, kEpiSwiglu, bf16, false, 2>(big, p, s);
        return launch_dl_sized<true, kEpiSwiglu, bf16>(big, p, s);
      case kOpGemm2:
        if (skip) return launch_dl_sized<false, kEpiStore, bf16, false, 1>(big, p, s);
        if (tskip) return launch_dl_sized<false, kEpiStore, bf16, false, 2>(big, p, s);
        return launch_dl_sized<false, kEpiStore, bf16>(big, p, s);
      default:
        break;
    }
  }
  // Data gradients from the weights as stored (k-major B) on the forward's
  // direct-to-LDS kernel: B ring, spread DMA, empty-block skip and split
  // last round as there, the B fragments read with transposing LDS reads
  // (DeepSeek-V3 shape: dgrad2 2.80 -> 1.68 ms, dgrad1 4.78 -> 3.31 ms
  // against the transposing-read backward kernel; Mixtral shape: the same
  // speed as from weights transposed once per step, whose transposes, 1 ms
  // per step, it saves). The k-tile offset rides in a 32-bit scalar, so
  // one part's k rows of one group's weights span under 2 GiB.
  if (!force_staged() && (op == kOpDgrad2 || op == kOpDgrad1) && p.ldb % 8 == 0 &&
      (long)(op == kOpDgrad1 ? p.K1 : p.K) * p.ldb * 2 <= INT_MAX) {
    if (op == kOpDgrad2 && p.K % 64 == 0) {
      if (skip)
        return launch_dl<256, 256, 2, 2, 4, false, kEpiSwigluBwd, bf16, false,
                         kSchedM, 0, 1, false, 3, true>(p, s);
      return big ? launch_dl<256, 256, 2, 2, 4, false, kEpiSwigluBwd, bf16, false,
                             kSchedM, 0, 2, false, 3, true>(p, s)
                 : launch_dl<128, 128, 2, 2, 2, false, kEpiSwigluBwd, bf16, false,
                             kSchedM, 0, 0, false, 0, true>(p, s);
    }
    if (op == kOpDgrad1 && p.K1 % 64 == 0 && p.K == 2 * p.K1) {
      if (skip)
        return launch_dl<256, 256, 2, 2, 4, false, kEpiStore, bf16, false,
                         kSchedM, 0, 1, true, 3, true>(p, s);
      if (big && p.slots != 0 && p.off) {  // split last round, as GEMM 2
        GemmParams q = p;
        if (q.slots < 0) q.slots = num_cus();
        hipError_t e = launch_dl<256, 256, 2, 2, 4, false, kEpiStore, bf16, false,
                                 kSchedM, 1, 2, true, 3, true>(q, s);
        if (e != hipSuccess) return e;
        return launch_dl<128, 128, 2, 2, 2, false, kEpiStore, bf16, false,
                         kSchedM, 2, 2, true, 0, true>(q, s);
      }
      return big ? launch_dl<256, 256, 2, 2, 4, false, kEpiStore, bf16, false,
                             kSchedM, 0, 2, true, 3, true>(p, s)
                 : launch_dl<128, 128, 2, 2, 2, false, kEpiStore, bf16, false,
                             kSchedM, 0, 0, true, 0, true>(p, s);
    }
  }
  // backward products on the direct-to-LDS kernel with k-major operands
  if (!force_staged()) {
    if (op == kOpWgrad && big && wgrad_persist())
    {
      // DMA from half the waves when the groups average 256 rows or more
      // (four k-steps and up per tile): the other half then passes each
      // barrier without waiting for its stores (weight gradients of
      // groups of ~550 to 2048 rows 5-8% faster). Groups of ~128 rows (two
      // k-steps per tile) measured 3-5% slower that way, the doubled DMA
      // issue of the loading waves no longer hidden between tiles.
      const int v = wgrad_persist();
      const bool half = v == 3 || (v == 1 && p.k_total >= 256L * (p.G > 0 ? p.G : 1));
      return v == 2 ? launch_wgrad<256, 256, 2, 4, false>(p, s)
             : half ? launch_wgrad<256, 256, 2, 4, true, 4>(p, s)
                    : launch_wgrad<256, 256, 2, 4>(p, s);
    }
    if (op == kOpWgrad)  // (the big form only for comparison)
      return !big ? launch_t<128, 128, 2, 2, true, true, kEpiStore, kSchedK>(p, s)
                  : launch_t<256, 256, 2, 4, true, true, kEpiStore, kSchedK>(p, s);
    // router backward: dx += d_logits Wr (Wr read k-major as stored), and
    // fp32 partial sums of d_logits^T x over token ranges
    if (op == kOpRouterDx)
      return launch_t<128, 128, 2, 2, false, true, kEpiAccum, kSchedM>(p, s);
    if (op == kOpRouterDw)
      return !big ? launch_t<128, 128, 2, 2, true, true, kEpiStoreF32, kSchedK>(p, s)
                  : launch_t<256, 256, 2, 4, true, true, kEpiStoreF32, kSchedK>(p, s);
  }
  if (op == kOpGemm1Mx)
    return skip || tskip
               ? launch_dl_sized<true, kEpiSwigluMx, bf16, true, 1>(big, p, s)
               : launch_dl_sized<true, kEpiSwigluMx, bf16, true>(big, p, s);
  if (op == kOpGemm1MxAct)
    return skip ? launch_dl_sized<true, kEpiSwiglu, bf16, true, 1>(big, p, s)
                : launch_dl_sized<true, kEpiSwiglu, bf16, true>(big, p, s);
  if (op == kOpDgrad2Mx)
    return launch_dl_sized<false, kEpiSwigluBwd, bf16, true>(big, p, s);
  if (op == kOpGemm2Mx)
    return launch_dl_sized<false, kEpiStore, bf16, true>(big, p, s);
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
    default:
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
