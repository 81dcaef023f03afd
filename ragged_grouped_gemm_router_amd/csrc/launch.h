// Internal launchers of the layer's non-GEMM kernels.
#pragma once

#include "common.h"

namespace moe {

// Copies handled by one histogram / ranking workgroup.
constexpr int kPermChunk = 1024;
// Most partial products a split router GEMM hands to the top-K kernels.
constexpr int kRouterMaxSplit = 8;

// Top-K gate over fp32 logits [T, E]. G > 1: `logits` holds G partial
// products [G, T, E] of a split router GEMM; they are summed in the order
// g = 0 .. G-1 into lout [T, E] and the gate runs on that sum.
hipError_t launch_topk(const float* logits, const float* bias, int T, int E,
                       int K, int gate, int32_t* idx, float* w,
                       hipStream_t s, int G = 1, float* lout = nullptr);

// Top-K fused with the permute's chunk ranking (E <= 32, K a divisor of
// kPermChunk with at least 64 tokens per chunk): idx, w as launch_topk,
// plus block_hist [nblk, E] (each chunk's expert counts, unscanned) and
// rank [T*K], as the histogram pass of launch_hist_rank_scan writes them.
bool topk_rank_supported(int E, int K);
hipError_t launch_topk_rank(const float* logits, const float* bias, int T,
                            int E, int K, int gate, int32_t* idx, float* w,
                            int32_t* block_hist, int32_t* rank, hipStream_t s,
                            int G = 1, float* lout = nullptr);

// Counting sort of the T*K copies by expert (stable in the copy index).
// block_hist: [nblk, E] int32 scratch, nblk = ceil(TK / kPermChunk), left
// holding the first slot of every (chunk, expert); rank: [TK] int32, each
// copy's rank among its chunk's copies of the same expert; tile_off:
// kNumTileBM arrays of E+1 (row-tile prefix per tile height). scan ==
// false stops after the histograms (block_hist then holds the counts of
// every (chunk, expert)), for launch_scatter to scan them itself.
// hist == false: block_hist and rank hold the histogram pass's results
// already (launch_topk_rank), and only the scan runs.
hipError_t launch_hist_rank_scan(const int32_t* idx, int TK, int E,
                                 int32_t* block_hist, int32_t* rank,
                                 int32_t* counts, int32_t* offsets,
                                 int32_t* const* tile_off, hipStream_t s,
                                 bool scan = true, bool hist = true);
// Whether the scatter can scan the chunk histograms itself (E * chunks
// small enough for one workgroup of the scatter).
bool scan_in_scatter(int TK, int E);
// tile_off[i][e] = sum_{e' < e} ceil(count_e' / kTileBM[i]) from offsets.
hipError_t launch_tile_prefix(const int32_t* offsets, int E,
                              int32_t* const* tile_off, hipStream_t s);
// dest / sorted_src of every copy from the sort above, and x_perm[dest[j]]
// = x[j / K] (row_bytes % 16 == 0). With counts given and
// scan_in_scatter(T * K, E), `first` holds the unscanned histograms, and
// the scatter scans them and writes counts, offsets and tile_off too.
hipError_t launch_scatter(const void* x, const int32_t* idx,
                          const int32_t* first, const int32_t* rank, int T,
                          int E, int K, long row_bytes, int32_t* dest,
                          int32_t* sorted_src, void* x_perm, hipStream_t s,
                          int32_t* counts = nullptr, int32_t* offsets = nullptr,
                          int32_t* const* tile_off = nullptr);
// dest / sorted_src only.
hipError_t launch_slots(const int32_t* idx, const int32_t* first,
                        const int32_t* rank, int TK, int E, int32_t* dest,
                        int32_t* sorted_src, hipStream_t s);
// out[t] = sum_k w[t,k] * y[dest[t*K+k]] (+ add[t]); w == NULL means 1.
hipError_t launch_combine(int dtype, const void* y, const int32_t* dest,
                          const float* w, const void* add, void* out, int T,
                          int K, int d, hipStream_t s);
// dy_perm[dest[t*K+k]] = w[t,k] * dy[t]; d_w[t,k] = <dy[t], y[dest[t*K+k]]>
hipError_t launch_combine_bwd(int dtype, const void* dy, const void* y,
                              const int32_t* dest, const float* w,
                              void* dy_perm, float* d_w, int T, int K, int d,
                              hipStream_t s);


// Router backward. d_logits [T,E] fp32 and the same in the activation
// dtype (d_logits_a, rows of ld_a elements, zero past E); split [G+1]
// token ranges for the partial sums.
hipError_t launch_router_grad(int dtype, const float* logits,
                              const int32_t* idx, const float* w,
                              const float* d_w, const int32_t* counts,
                              float aux_coef, int T, int E, int K, int gate,
                              float* d_logits, void* d_logits_a, int ld_a,
                              int G, int32_t* split, hipStream_t s);
// Balance statistics: f = counts / T, p_mean = mean gate probability,
// aux = E sum f p_mean, through G token-range partial sums in part [G, E].
hipError_t launch_balance_stats(const float* logits, const int32_t* counts,
                                int T, int E, int gate, int G, float* part,
                                float* f, float* p_mean, float* aux,
                                hipStream_t s);
// split[g] = g * T / G for g = 0..G (G <= 1023).
hipError_t launch_split(int T, int G, int32_t* split, hipStream_t s);
// Route-bias balance step and load monitor (one block each, E <= 1024).
hipError_t launch_bias_update(const int32_t* counts, int E, float gamma,
                              float target, int rule, float* bias,
                              float* load, hipStream_t s);
hipError_t launch_balance_monitor(const float* hist, int W, int E, float* out,
                                  hipStream_t s);
// out[i] = sum_{g < G} part[g * n + i] (fixed order), in dtype.
hipError_t launch_reduce_parts(int dtype, const float* part, long n, int G,
                               void* out, hipStream_t s);
// y += x elementwise (n % 8 == 0).
hipError_t launch_add_inplace(int dtype, void* y, const void* x, long n,
                              hipStream_t s);

// MXFP8 (E4M3 elements, E8M0 scale per 32 along rows). Every scale array
// is in the span-grouped layout of mx_scale_index: [cols/128][rows][4] for
// an operand of `rows` rows; a pointer "offset to column c" (c a multiple
// of 128) is the array's start plus c / 128 * rows * 4.
// Rows of a contiguous bf16 [rows, cols] into codes at q + r * ldq and the
// scales of the rows-row operand (q, scales offset to the first column).
hipError_t launch_quantize_mxfp8_strided(const void* src, long rows,
                                         long cols, uint8_t* q, long ldq,
                                         uint8_t* scales, hipStream_t s);
// Codes [rows, cols] + scales -> bf16 [rows, cols].
hipError_t launch_dequantize_mxfp8(const uint8_t* q, const uint8_t* scales,
                                   long rows, long cols, void* out,
                                   hipStream_t s);
// Per batch: bf16 [R, C] -> codes [C, ldq] (blocks along R, batch stride
// C * ldq) and the scales of the stacked [batch * C, ldq] operand; q and
// scales offset to the first destination column. R % 32 == 0, C % 64 == 0.
hipError_t launch_quantize_mxfp8_cols(const void* src, long batch, int R,
                                      int C, uint8_t* q, long ldq,
                                      uint8_t* scales, hipStream_t s);
// Rows of a contiguous bf16 [rows, cols] (cols % 128 == 0) into codes
// [rows, cols] and scales.
hipError_t launch_quantize_mxfp8(const void* src, long rows, long cols,
                                 uint8_t* q, uint8_t* scales, hipStream_t s);
// x [T, d] quantised into the T*K rows of x_perm at dest (codes, scales).
hipError_t launch_scatter_rows_mxfp8(const void* x, int T, int K, int d,
                                     const int32_t* dest, uint8_t* xq,
                                     uint8_t* xs, hipStream_t s);

}  // namespace moe
