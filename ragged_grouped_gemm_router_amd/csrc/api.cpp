// C ABI of the MoE layer: argument validation, workspace carving and the
// launch sequence of each entry point. No allocation, no synchronisation,
// no state kept between calls.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gemm.h"
#include "launch.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;
constexpr long kMaxCopies = 1L << 30;  // int32 slots with headroom

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
size_t act_bytes(int dt) { return dt == MOE_F32 ? 4 : 2; }
long cdiv(long a, long b) { return (a + b - 1) / b; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

moe_status check_desc(const moe_desc* d) {
  if (!d) return MOE_EINVAL;
  if (d->T < 0 || d->d_model <= 0 || d->d_ff <= 0 || d->E <= 0 || d->K <= 0 ||
      d->d_ff_shared < 0)
    return MOE_EINVAL;
  if (d->K > d->E) return MOE_EINVAL;
  if (d->gate != MOE_GATE_SOFTMAX && d->gate != MOE_GATE_SIGMOID) return MOE_EINVAL;
  if (d->act_dtype != MOE_F32 && d->act_dtype != MOE_BF16) return MOE_EINVAL;
  if (d->flags & ~(MOE_FLAG_SAVE_ACTS | MOE_FLAG_NO_TAIL_SPLIT)) return MOE_EINVAL;
  if (d->K > MOE_K_MAX || d->E > MOE_E_MAX) return MOE_EUNSUPPORTED;
  if (d->gemm_dtype != d->act_dtype &&
      !(d->gemm_dtype == MOE_MXFP8 && d->act_dtype == MOE_BF16))
    return MOE_EINVAL;
  if (d->d_model % 8 || d->d_ff % 8 || d->d_ff_shared % 8) return MOE_EUNSUPPORTED;
  if (d->gemm_dtype == MOE_MXFP8) {
    // whole 128-element k-tiles for every GEMM
    if (d->d_model % 128 || d->d_ff % 128 || d->d_ff_shared % 128)
      return MOE_EUNSUPPORTED;
  }
  if ((long)d->T * d->K > kMaxCopies) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Forward scratch: permute histogram, tile prefixes, shared-expert hidden,
// the split router GEMM's partial products.
struct FwdWs {
  float* router_part;  // [router_split.G, T, E] fp32 when G > 1
  int32_t* block_hist;
  int32_t* rank;
  uint8_t* xq;  // MXFP8: x quantised once (shared expert, gathered GEMM 1):
  uint8_t* xs;  // codes [T, d] and E8M0 scales [T, d/32]
  int32_t* tile_off[kNumTileBM];
  void* h_shared;
};
struct BwdWs {
  int32_t* tile_off[kNumTileBM];
  void* dy_perm;
  void* da;
  void* db;
  void* dx_perm;
  // shared expert: recomputed a, b (then da, db in place), h, its share of
  // dx, and the one-group row range [0, T)
  void* sa;
  void* sb;
  void* sh;
  void* sdx;
  int32_t* srange;
  // MXFP8: dy_perm and [da | db] quantised, h dequantised for dW2
  uint8_t* dyq;
  uint8_t* dys;
  uint8_t* dgq;
  uint8_t* dgs;
  void* h_bf;
  // MXFP8 shared expert: x and dy quantised, its h (codes, scales) and
  // [da | db] quantised, x dequantised for its weight gradients
  uint8_t* sxq;
  uint8_t* sxs;
  uint8_t* sdyq;
  uint8_t* sdys;
  uint8_t* shq;
  uint8_t* shs;
  uint8_t* sdgq;
  uint8_t* sdgs;
  void* sx_bf;
};

bool force_simt();

// The router GEMM inside the whole forward, bf16 on the direct-to-LDS
// kernel: its contraction over d_model is split into G ranges of kmul
// columns (whole k-tiles of 64) whose partial products the top-K kernel
// sums in order. G brings the launch to about kRouterWgs workgroups (one
// per CU for the 64 x 256 tile, two for the smaller ones; a fixed count,
// so that G, the workspace and the logits' rounding depend on the
// descriptor alone), at most kRouterMaxSplit splits and kRouterPartBytes of
// partials.
// G = 1: one range of all d_model columns.
constexpr long kRouterWgs = 256;
constexpr size_t kRouterPartBytes = (size_t)32 << 20;
struct RouterSplit {
  int G, kmul;
};
RouterSplit router_split(const moe_desc* d) {
  RouterSplit r{1, d->d_model};
  if (d->act_dtype != MOE_BF16 || d->d_model % 64 || d->T <= 0 ||
      force_simt() || !gemm_direct_ok())
    return r;
  const int bm = d->E <= 32 ? 32 : 64;
  const int bn = d->E <= 32 ? 32 : d->E <= 64 ? 64 : 256;
  const long tiles = cdiv(d->T, bm) * cdiv(d->E, bn);
  const long target = bn == 256 ? kRouterWgs : 2 * kRouterWgs;
  const int kt = d->d_model / 64;
  long G = (target + tiles / 2) / tiles;
  const long part = (long)d->T * d->E * (long)sizeof(float);
  G = std::min<long>({G, (long)kRouterMaxSplit, (long)kt,
                      (long)(kRouterPartBytes / part)});
  if (G <= 1) return r;
  const int per = (int)cdiv(kt, G);  // k-tiles per split
  r.G = (int)cdiv(kt, per);
  r.kmul = per * 64;
  return r;
}

size_t fwd_ws_layout(const moe_desc* d, char* base, FwdWs* w) {
  const long TK = (long)d->T * d->K;
  const long nblk = cdiv(TK, kPermChunk);
  size_t o = 0;
  const RouterSplit rs = router_split(d);
  if (w) w->router_part = rs.G > 1 ? (float*)(base + o) : nullptr;
  if (rs.G > 1) o = align_up(o + sizeof(float) * (size_t)rs.G * d->T * d->E);
  if (w) w->block_hist = (int32_t*)(base + o);
  o = align_up(o + sizeof(int32_t) * (size_t)(d->E * (nblk > 0 ? nblk : 1)));
  if (w) w->rank = (int32_t*)(base + o);
  o = align_up(o + sizeof(int32_t) * (size_t)(TK > 0 ? TK : 1));
  for (int i = 0; i < kNumTileBM; ++i) {
    if (w) w->tile_off[i] = (int32_t*)(base + o);
    o = align_up(o + sizeof(int32_t) * (size_t)(d->E + 1));
  }
  if (w) w->h_shared = base + o;
  o = align_up(o + act_bytes(d->act_dtype) * (size_t)d->T * d->d_ff_shared);
  if (d->gemm_dtype == MOE_MXFP8) {
    const size_t n = (size_t)d->T * d->d_model;
    if (w) w->xq = (uint8_t*)(base + o);
    o = align_up(o + n);
    if (w) w->xs = (uint8_t*)(base + o);
    o = align_up(o + n / 32);
  }
  return o;
}

size_t bwd_ws_layout(const moe_desc* d, char* base, BwdWs* w) {
  const size_t TK = (size_t)d->T * d->K, b = act_bytes(d->act_dtype);
  size_t o = 0;
  for (int i = 0; i < kNumTileBM; ++i) {
    if (w) w->tile_off[i] = (int32_t*)(base + o);
    o = align_up(o + sizeof(int32_t) * (size_t)(d->E + 1));
  }
  if (w) w->dy_perm = base + o;
  o = align_up(o + b * TK * d->d_model);
  if (w) w->da = base + o;
  o = align_up(o + b * TK * d->d_ff);
  if (w) w->db = base + o;
  o = align_up(o + b * TK * d->d_ff);
  if (w) w->dx_perm = base + o;
  o = align_up(o + b * TK * d->d_model);
  if (d->d_ff_shared > 0) {
    const size_t T = d->T, fs = d->d_ff_shared;
    void** bufs[3] = {w ? &w->sa : nullptr, w ? &w->sb : nullptr,
                      w ? &w->sh : nullptr};
    for (void** q : bufs) {
      if (q) *q = base + o;
      o = align_up(o + b * T * fs);
    }
    if (w) w->sdx = base + o;
    o = align_up(o + b * T * d->d_model);
    if (w) w->srange = (int32_t*)(base + o);
    o = align_up(o + 2 * sizeof(int32_t));
  }
  if (d->gemm_dtype == MOE_MXFP8) {
    const size_t dm = d->d_model, f = d->d_ff;
    uint8_t** u8s[4] = {w ? &w->dyq : nullptr, w ? &w->dys : nullptr,
                        w ? &w->dgq : nullptr, w ? &w->dgs : nullptr};
    const size_t n[4] = {TK * dm, TK * dm / 32, TK * 2 * f, TK * 2 * f / 32};
    for (int i = 0; i < 4; ++i) {
      if (u8s[i]) *u8s[i] = (uint8_t*)(base + o);
      o = align_up(o + n[i]);
    }
    if (w) w->h_bf = base + o;
    o = align_up(o + b * TK * f);
    if (d->d_ff_shared > 0) {
      const size_t T = d->T, fs = d->d_ff_shared;
      uint8_t** q[8] = {w ? &w->sxq : nullptr,  w ? &w->sxs : nullptr,
                        w ? &w->sdyq : nullptr, w ? &w->sdys : nullptr,
                        w ? &w->shq : nullptr,  w ? &w->shs : nullptr,
                        w ? &w->sdgq : nullptr, w ? &w->sdgs : nullptr};
      const size_t m[8] = {T * dm, T * dm / 32, T * dm, T * dm / 32,
                           T * fs, T * fs / 32, T * 2 * fs, T * 2 * fs / 32};
      for (int i = 0; i < 8; ++i) {
        if (q[i]) *q[i] = (uint8_t*)(base + o);
        o = align_up(o + m[i]);
      }
      if (w) w->sx_bf = base + o;
      o = align_up(o + b * T * dm);
    }
  }
  return o;
}

bool force_simt() {
  static const int v = [] {
    const char* s = tuning_env("MOE_GEMM_BACKEND");
    return (s && strcmp(s, "simt") == 0) ? 1 : 0;
  }();
  return v != 0;
}

GemmParams gp() {
  GemmParams p;
  memset(&p, 0, sizeof(p));
  p.K1 = INT_MAX;
  p.G = 1;
  return p;
}

hipError_t run_gemm(GemmOp op, int dtype, GemmParams p,
                    int32_t* const* tile_off, hipStream_t s) {
  // the router's backward products are small and always run on SIMT
  const bool router_bwd = op == kOpRouterDx || op == kOpRouterDw;
  if (dtype == MOE_BF16 && !force_simt() && !router_bwd && mfma_supported(op, p))
    return gemm_mfma(op, p, tile_off, s);
  if (op != kOpWgrad && op != kOpRouterDw) {
    if (p.off) {
      p.tile_off = tile_off[tile_bm_slot(kSimtBM)];
      p.tiles_m_max = (int)(cdiv(p.M, kSimtBM) + (p.G < p.M ? p.G : p.M));
    } else {
      p.tiles_m_max = (int)cdiv(p.M, kSimtBM);
    }
  }
  return gemm_simt(op, dtype, p, s);
}

void record(void* ev, hipStream_t s) {
  if (ev) (void)hipEventRecord((hipEvent_t)ev, s);
}

// --- building blocks shared by the entry points --------------------------
// ws != NULL (the whole forward): where the shape allows, the top-K kernel
// also ranks the permute's chunks into ws (see launch_topk_rank), and
// *ranked says so.
hipError_t do_route(const moe_desc* d, const void* x, const void* wr,
                    const float* bias, const float* logits_in,
                    float* logits_out, int32_t* idx, float* w, hipStream_t s,
                    const FwdWs* ws = nullptr, bool* ranked = nullptr) {
  const float* L = logits_in;
  int G = 1;  // partial products of the split router GEMM in L
  if (!L) {
    // (a forward's workspace holds the partials of a split; on its own
    // the router GEMM runs as one contraction)
    const RouterSplit rs = ws ? router_split(d) : RouterSplit{1, d->d_model};
    GemmParams p = gp();
    p.M = d->T; p.N = d->E; p.K = d->d_model;
    p.A = x; p.lda = d->d_model;
    p.B = wr; p.ldb = d->d_model;
    p.C = logits_out; p.ldc = d->E;
    p.G = rs.G; p.kmul = rs.kmul;
    if (rs.G > 1) {
      G = rs.G;
      p.C = ws->router_part;
      p.sC = (long)d->T * d->E;
    }
    hipError_t e = run_gemm(kOpRouter, d->act_dtype, p, nullptr, s);
    if (e != hipSuccess) return e;
    L = G > 1 ? ws->router_part : logits_out;
  }
  if (ranked) *ranked = false;
  // (the fused kernel moves logits rows in 16-byte pieces)
  const bool al16 = ((uintptr_t)L & 15) == 0 &&
                    (G == 1 || ((uintptr_t)logits_out & 15) == 0);
  if (ws && ranked && al16 && topk_rank_supported(d->E, d->K)) {
    *ranked = true;
    return launch_topk_rank(L, bias, d->T, d->E, d->K, d->gate, idx, w,
                            ws->block_hist, ws->rank, s, G, logits_out);
  }
  return launch_topk(L, bias, d->T, d->E, d->K, d->gate, idx, w, s, G,
                     logits_out);
}

// x_perm == NULL: only the indices (the expert GEMM gathers its rows from
// x; under MXFP8 x is quantised once into the workspace for it).
// ranked: the top-K kernel wrote the chunk histograms and ranks already.
hipError_t do_permute(const moe_desc* d, const void* x, const int32_t* idx,
                      int32_t* counts, int32_t* offsets, int32_t* src,
                      int32_t* dest, void* x_perm, uint8_t* x_perm_scales,
                      const FwdWs& ws, hipStream_t s, bool ranked = false) {
  const int TK = d->T * d->K;
  // materialised bf16/fp32 rows with few experts: the scatter scans the
  // chunk histograms itself (one launch fewer)
  const bool fused = x_perm && d->gemm_dtype != MOE_MXFP8 &&
                     scan_in_scatter(TK, d->E);
  hipError_t e = launch_hist_rank_scan(idx, TK, d->E, ws.block_hist, ws.rank,
                                       counts, offsets, ws.tile_off, s, !fused,
                                       !ranked);
  if (e != hipSuccess) return e;
  if (!x_perm) {
    e = launch_slots(idx, ws.block_hist, ws.rank, TK, d->E, dest, src, s);
    if (e != hipSuccess || d->gemm_dtype != MOE_MXFP8) return e;
    return launch_quantize_mxfp8(x, d->T, d->d_model, ws.xq, ws.xs, s);
  }
  if (d->gemm_dtype == MOE_MXFP8) {
    e = launch_slots(idx, ws.block_hist, ws.rank, TK, d->E, dest, src, s);
    if (e != hipSuccess) return e;
    return launch_scatter_rows_mxfp8(x, d->T, d->K, d->d_model, dest,
                                     (uint8_t*)x_perm, x_perm_scales, s);
  }
  return launch_scatter(x, idx, ws.block_hist, ws.rank, d->T, d->E, d->K,
                        (long)d->d_model * act_bytes(d->act_dtype), dest, src,
                        x_perm, s, fused ? counts : nullptr,
                        fused ? offsets : nullptr, ws.tile_off);
}

hipError_t do_gemm1(const moe_desc* d, const void* A, const int32_t* off,
                    int rows, int G, const void* w1, const void* w3, int f,
                    void* h, void* a_out, void* b_out, int32_t* const* toff,
                    hipStream_t s, const int32_t* gsrc = nullptr) {
  GemmParams p = gp();
  p.M = rows; p.N = f; p.K = d->d_model; p.G = G; p.off = off;
  p.A = A; p.lda = d->d_model;
  p.gsrc = gsrc; p.gdiv = d->K;
  p.B = w1; p.B2 = w3; p.ldb = d->d_model; p.sB = (long)f * d->d_model;
  p.C = h; p.C2 = a_out; p.C3 = b_out; p.ldc = f;
  p.slots = d->flags & MOE_FLAG_NO_TAIL_SPLIT ? 0 : -1;
  return run_gemm(kOpGemm1, d->act_dtype, p, toff, s);
}

hipError_t do_gemm2(const moe_desc* d, const void* h, const int32_t* off,
                    int rows, int G, const void* w2, int f, void* y,
                    int32_t* const* toff, hipStream_t s) {
  GemmParams p = gp();
  p.M = rows; p.N = d->d_model; p.K = f; p.G = G; p.off = off;
  p.A = h; p.lda = f;
  p.B = w2; p.ldb = f; p.sB = (long)d->d_model * f;
  p.C = y; p.ldc = d->d_model;
  p.slots = d->flags & MOE_FLAG_NO_TAIL_SPLIT ? 0 : -1;
  return run_gemm(kOpGemm2, d->act_dtype, p, toff, s);
}

// MXFP8 expert GEMMs. h lives in the caller's h buffer as E4M3 codes
// [T*K, d_ff] followed by their E8M0 scales (span-grouped, T*K rows).
// With a shared expert, x is quantised into the workspace and the shared
// GEMMs run as one dense group, h_shared holding codes then scales.
// gsrc != NULL: x_perm was not written; GEMM 1 gathers the rows of the
// quantised x in the workspace through gsrc (sorted_src).
hipError_t do_experts_mx(const moe_desc* d, const void* x_perm,
                         const uint8_t* x_perm_scales, const int32_t* offsets,
                         const moe_expert_weights* rw, const void* x_shared,
                         const moe_expert_weights* sw, void* h, void* y_perm,
                         void* y_shared, const FwdWs& ws, hipStream_t s,
                         void* ev_mid, const int32_t* gsrc = nullptr,
                         void* act_a = nullptr, void* act_b = nullptr) {
  const int TK = d->T * d->K, dm = d->d_model, f = d->d_ff;
  uint8_t* hq = (uint8_t*)h;
  uint8_t* hs = hq + (size_t)TK * f;
  GemmParams p = gp();
  p.M = TK; p.N = f; p.K = dm; p.G = d->E; p.off = offsets;
  p.A = gsrc ? ws.xq : x_perm; p.lda = dm;
  p.As = gsrc ? ws.xs : x_perm_scales;
  p.gsrc = gsrc; p.gdiv = d->K;
  p.B = rw->w1; p.B2 = rw->w3; p.ldb = dm; p.sB = (long)f * dm;
  p.Bs = rw->w1_scales; p.B2s = rw->w3_scales;
  p.s_rows = gsrc ? d->T : TK;
  p.C = hq; p.C2 = hs; p.ldc = f;
  p.Sa = act_a; p.Sb = act_b;
  hipError_t e = gemm_mfma(kOpGemm1Mx, p, ws.tile_off, s);
  if (e != hipSuccess) return e;
  record(ev_mid, s);
  p = gp();
  p.M = TK; p.N = dm; p.K = f; p.G = d->E; p.off = offsets;
  p.A = hq; p.lda = f; p.As = hs;
  p.B = rw->w2; p.ldb = f; p.sB = (long)dm * f;
  p.Bs = rw->w2_scales; p.s_rows = TK;
  p.C = y_perm; p.ldc = dm;
  p.slots = d->flags & MOE_FLAG_NO_TAIL_SPLIT ? 0 : -1;
  e = gemm_mfma(kOpGemm2Mx, p, ws.tile_off, s);
  if (e != hipSuccess || !x_shared || d->d_ff_shared == 0) return e;
  const int T = d->T, fs = d->d_ff_shared;
  if (!gsrc) {  // (with gathered rows x is quantised already)
    e = launch_quantize_mxfp8(x_shared, T, dm, ws.xq, ws.xs, s);
    if (e != hipSuccess) return e;
  }
  uint8_t* sq = (uint8_t*)ws.h_shared;
  uint8_t* ss = sq + (size_t)T * fs;
  p = gp();
  p.M = T; p.N = fs; p.K = dm;
  p.A = ws.xq; p.lda = dm; p.As = ws.xs;
  p.B = sw->w1; p.B2 = sw->w3; p.ldb = dm;
  p.Bs = sw->w1_scales; p.B2s = sw->w3_scales; p.s_rows = T;
  p.C = sq; p.C2 = ss; p.ldc = fs;
  e = gemm_mfma(kOpGemm1Mx, p, ws.tile_off, s);
  if (e != hipSuccess) return e;
  p = gp();
  p.M = T; p.N = dm; p.K = fs;
  p.A = sq; p.lda = fs; p.As = ss;
  p.B = sw->w2; p.ldb = fs;
  p.Bs = sw->w2_scales; p.s_rows = T;
  p.C = y_shared; p.ldc = dm;
  return gemm_mfma(kOpGemm2Mx, p, ws.tile_off, s);
}

// MX scale arrays are read and written a 4-code word at a time.
bool scale_ptr_ok(const void* p) {
  return p && ((uintptr_t)p & 3) == 0;
}

bool mx_weights_ok(const moe_expert_weights* w) {
  return w && w->w1 && w->w3 && w->w2 && scale_ptr_ok(w->w1_scales) &&
         scale_ptr_ok(w->w3_scales) && scale_ptr_ok(w->w2_scales);
}

// gsrc != NULL: x_perm is x itself and GEMM 1 gathers its rows through
// gsrc (sorted_src).
hipError_t do_experts(const moe_desc* d, const void* x_perm,
                      const int32_t* offsets, const moe_expert_weights* rw,
                      const void* x_shared, const moe_expert_weights* sw,
                      void* h, void* y_perm, void* y_shared, void* act_a,
                      void* act_b, const FwdWs& ws, hipStream_t s,
                      void* ev_mid, const int32_t* gsrc = nullptr) {
  const int TK = d->T * d->K;
  hipError_t e = do_gemm1(d, x_perm, offsets, TK, d->E, rw->w1, rw->w3,
                          d->d_ff, h, act_a, act_b, ws.tile_off, s, gsrc);
  if (e != hipSuccess) return e;
  record(ev_mid, s);
  e = do_gemm2(d, h, offsets, TK, d->E, rw->w2, d->d_ff, y_perm, ws.tile_off, s);
  if (e != hipSuccess) return e;
  if (x_shared && d->d_ff_shared > 0) {
    e = do_gemm1(d, x_shared, nullptr, d->T, 1, sw->w1, sw->w3,
                 d->d_ff_shared, ws.h_shared, nullptr, nullptr, ws.tile_off, s);
    if (e != hipSuccess) return e;
    e = do_gemm2(d, ws.h_shared, nullptr, d->T, 1, sw->w2, d->d_ff_shared,
                 y_shared, ws.tile_off, s);
  }
  return e;
}

bool weights_ok(const moe_expert_weights* w) {
  return w && w->w1 && w->w3 && w->w2;
}

// MXFP8 backward (validated by moe_backward): the data-gradient products on
// MX operands, the weight gradients in bf16 from the forward's operands.
hipError_t do_backward_mx(const moe_desc* d, const moe_bwd_args* a, void* ws,
                          hipStream_t s) {
  BwdWs w;
  bwd_ws_layout(d, (char*)ws, &w);
  const int TK = d->T * d->K, dm = d->d_model, f = d->d_ff, E = d->E;
  hipError_t e;
#define MOE_TRY(x)                        \
  do {                                    \
    e = (x);                              \
    if (e != hipSuccess) return e;        \
  } while (0)
  record(a->events[0], s);
  MOE_TRY(launch_tile_prefix(a->offsets, E, w.tile_off, s));
  MOE_TRY(launch_combine_bwd(MOE_BF16, a->dy, a->y_perm, a->dest, a->topk_w,
                             w.dy_perm, a->d_topk_w, d->T, d->K, dm, s));
  MOE_TRY(launch_quantize_mxfp8(w.dy_perm, TK, dm, w.dyq, w.dys, s));
  const bool shared = d->d_ff_shared > 0;
  const int T = d->T, fs = d->d_ff_shared;
  if (shared) {  // x and the (ungated) dy of the shared expert, quantised
    MOE_TRY(launch_quantize_mxfp8(a->x, T, dm, w.sxq, w.sxs, s));
    MOE_TRY(launch_quantize_mxfp8(a->dy, T, dm, w.sdyq, w.sdys, s));
  }
  record(a->events[1], s);
  // a, b of the forward: saved, or GEMM 1 again on its MX operands (bf16)
  const void* sa = a->act_a;
  const void* sb = a->act_b;
  if (!sa) {
    sa = w.da;
    sb = w.db;
    GemmParams p = gp();
    p.M = TK; p.N = f; p.K = dm; p.G = E; p.off = a->offsets;
    p.A = a->x_perm; p.lda = dm; p.As = a->x_perm_scales;
    p.B = a->routed.w1; p.B2 = a->routed.w3; p.ldb = dm; p.sB = (long)f * dm;
    p.Bs = a->routed.w1_scales; p.B2s = a->routed.w3_scales;
    p.s_rows = TK;
    p.C = nullptr; p.C2 = w.da; p.C3 = w.db; p.ldc = f;
    MOE_TRY(gemm_mfma(kOpGemm1MxAct, p, w.tile_off, s));
  }
  if (shared) {  // its a, b (bf16) and MX h, as the forward made them
    MOE_TRY(launch_split(T, 1, w.srange, s));
    GemmParams p = gp();
    p.M = T; p.N = fs; p.K = dm;
    p.A = w.sxq; p.lda = dm; p.As = w.sxs;
    p.B = a->shared.w1; p.B2 = a->shared.w3; p.ldb = dm;
    p.Bs = a->shared.w1_scales; p.B2s = a->shared.w3_scales; p.s_rows = T;
    p.C = w.shq; p.C2 = w.shs; p.ldc = fs;
    p.Sa = w.sa; p.Sb = w.sb;
    MOE_TRY(gemm_mfma(kOpGemm1Mx, p, w.tile_off, s));
  }
  record(a->events[2], s);
  {  // dh = Q(dy_perm) W2t_e, then (da, db) in place of (a, b)
    GemmParams p = gp();
    p.M = TK; p.N = f; p.K = dm; p.G = E; p.off = a->offsets;
    p.A = w.dyq; p.lda = dm; p.As = w.dys;
    p.B = a->w2t; p.ldb = dm; p.sB = (long)f * dm;
    p.Bs = a->w2t_scales; p.s_rows = TK;
    p.C = w.da; p.C2 = w.db; p.ldc = f;
    p.aux_a = sa; p.aux_b = sb;
    MOE_TRY(gemm_mfma(kOpDgrad2Mx, p, w.tile_off, s));
    // [da | db] quantised along d_ff, side by side
    // (db's scales start at column f: f / 128 spans of TK rows)
    MOE_TRY(launch_quantize_mxfp8_strided(w.da, TK, f, w.dgq, 2L * f, w.dgs,
                                          s));
    MOE_TRY(launch_quantize_mxfp8_strided(w.db, TK, f, w.dgq + f, 2L * f,
                                          w.dgs + (long)TK * f / 32, s));
  }
  if (shared) {  // dh_s = Q(dy) Ws2t, (da_s, db_s) in place, quantised
    GemmParams p = gp();
    p.M = T; p.N = fs; p.K = dm;
    p.A = w.sdyq; p.lda = dm; p.As = w.sdys;
    p.B = a->ws2t; p.ldb = dm; p.Bs = a->ws2t_scales; p.s_rows = T;
    p.C = w.sa; p.C2 = w.sb; p.ldc = fs;
    p.aux_a = w.sa; p.aux_b = w.sb;
    MOE_TRY(gemm_mfma(kOpDgrad2Mx, p, w.tile_off, s));
    MOE_TRY(launch_quantize_mxfp8_strided(w.sa, T, fs, w.sdgq, 2L * fs, w.sdgs,
                                          s));
    MOE_TRY(launch_quantize_mxfp8_strided(w.sb, T, fs, w.sdgq + fs, 2L * fs,
                                          w.sdgs + (long)T * fs / 32, s));
  }
  record(a->events[3], s);
  {  // dx_perm = Q([da | db]) W13t_e
    GemmParams p = gp();
    p.M = TK; p.N = dm; p.K = 2 * f; p.G = E; p.off = a->offsets;
    p.A = w.dgq; p.lda = 2 * f; p.As = w.dgs;
    p.B = a->w13t; p.ldb = 2 * f; p.sB = (long)dm * 2 * f;
    p.Bs = a->w13t_scales; p.s_rows = TK;
    p.C = w.dx_perm; p.ldc = dm;
    p.slots = d->flags & MOE_FLAG_NO_TAIL_SPLIT ? 0 : -1;
    MOE_TRY(gemm_mfma(kOpGemm2Mx, p, w.tile_off, s));
  }
  if (shared) {  // dx_s = Q([da_s | db_s]) Ws13t
    GemmParams p = gp();
    p.M = T; p.N = dm; p.K = 2 * fs;
    p.A = w.sdgq; p.lda = 2 * fs; p.As = w.sdgs;
    p.B = a->ws13t; p.ldb = 2 * fs; p.Bs = a->ws13t_scales; p.s_rows = T;
    p.C = w.sdx; p.ldc = dm;
    MOE_TRY(gemm_mfma(kOpGemm2Mx, p, w.tile_off, s));
  }
  record(a->events[4], s);
  MOE_TRY(launch_combine(MOE_BF16, w.dx_perm, a->dest, nullptr,
                         shared ? w.sdx : nullptr, a->dx, d->T, d->K, dm, s));
  record(a->events[5], s);
  // weight gradients in bf16, as in the bf16 backward
  {  // dW2_e = dy_perm^T h, h dequantised from the forward's codes
    const uint8_t* hq = (const uint8_t*)a->h;
    MOE_TRY(launch_dequantize_mxfp8(hq, hq + (size_t)TK * f, TK, f, w.h_bf, s));
    GemmParams p = gp();
    p.M = dm; p.N = f; p.G = E; p.off = a->offsets; p.k_total = TK;
    p.A = w.dy_perm; p.lda = dm;
    p.B = w.h_bf; p.ldb = f;
    p.C = a->dw2; p.ldc = f; p.sC = (long)dm * f;
    MOE_TRY(run_gemm(kOpWgrad, MOE_BF16, p, w.tile_off, s));
  }
  if (shared) {  // dWs2 = dy^T h_s, h_s dequantised; x dequantised too
    MOE_TRY(launch_dequantize_mxfp8(w.shq, w.shs, T, fs, w.sh, s));
    MOE_TRY(launch_dequantize_mxfp8(w.sxq, w.sxs, T, dm, w.sx_bf, s));
    GemmParams p = gp();
    p.M = dm; p.N = fs; p.G = 1; p.off = w.srange; p.k_total = d->T;
    p.A = a->dy; p.lda = dm;
    p.B = w.sh; p.ldb = fs;
    p.C = a->dws2; p.ldc = fs;
    MOE_TRY(run_gemm(kOpWgrad, MOE_BF16, p, w.tile_off, s));
  }
  record(a->events[6], s);
  // dW1_e = da^T x_perm, dW3_e = db^T x_perm, x_perm dequantised (into the
  // dx_perm buffer, free after the gather-sum)
  MOE_TRY(launch_dequantize_mxfp8((const uint8_t*)a->x_perm, a->x_perm_scales,
                                  TK, dm, w.dx_perm, s));
  for (int which = 0; which < 2; ++which) {
    GemmParams p = gp();
    p.M = f; p.N = dm; p.G = E; p.off = a->offsets; p.k_total = TK;
    p.A = which ? w.db : w.da; p.lda = f;
    p.B = w.dx_perm; p.ldb = dm;
    p.C = which ? a->dw3 : a->dw1; p.ldc = dm; p.sC = (long)f * dm;
    MOE_TRY(run_gemm(kOpWgrad, MOE_BF16, p, w.tile_off, s));
    if (shared) {  // dWs1 = da_s^T x, dWs3 = db_s^T x (x as quantised)
      GemmParams q = gp();
      q.M = fs; q.N = dm; q.G = 1; q.off = w.srange; q.k_total = d->T;
      q.A = which ? w.sb : w.sa; q.lda = fs;
      q.B = w.sx_bf; q.ldb = dm;
      q.C = which ? a->dws3 : a->dws1; q.ldc = dm;
      MOE_TRY(run_gemm(kOpWgrad, MOE_BF16, q, w.tile_off, s));
    }
  }
  record(a->events[7], s);
#undef MOE_TRY
  return hipSuccess;
}

}  // namespace

// ===========================================================================
// Router backward workspace: d_logits in the activation dtype [T, E], the
// token-range partial sums of the router-weight gradient [G, E, d] fp32,
// the G + 1 range bounds, and the router's share of dx [T, d].
struct RouterWs {
  void* dl_a;    // d_logits in the activation dtype, [T, ld_dl], zero padded
  float* part;   // [G, E, d_model] token-range partial sums of d Wr
  int32_t* split;
  void* dx_router;
  float* bpart;  // balance statistics: [Gb, E] token-range partial sums
  int G, Gb, ld_dl;
};

// Token ranges of the router-weight gradient: enough (tile, range) pairs
// to cover the CUs about four times, ranges of at least 256 tokens, and
// at most half as many bytes of fp32 partial sums as the x they read.
int router_splits(const moe_desc* d) {
  const long T = d->T, E = d->E, dm = d->d_model;
  const long tiles = ((E + 127) / 128) * ((dm + 127) / 128);
  long G = 1024 / (tiles > 0 ? tiles : 1);
  G = std::min(G, T / 256);
  G = std::min(G, T / (4 * E));
  return (int)std::max(1L, std::min(G, 64L));
}

// token ranges of the balance statistics: about 32 tokens each, so that
// even a few thousand tokens spread over every CU
int balance_splits(int T) {
  const int G = (T + 31) / 32;
  return G < 1 ? 1 : (G > 1024 ? 1024 : G);
}

size_t router_ws_layout(const moe_desc* d, char* base, RouterWs* w) {
  const size_t b = act_bytes(d->act_dtype), T = d->T, E = d->E,
               dm = d->d_model;
  const int G = router_splits(d);
  const size_t ld_dl = (E + 63) / 64 * 64;
  size_t o = 0;
  if (w) { w->dl_a = base + o; w->G = G; w->ld_dl = (int)ld_dl; }
  o = align_up(o + b * T * ld_dl);
  if (w) w->part = (float*)(base + o);
  o = align_up(o + sizeof(float) * (size_t)G * E * dm);
  if (w) w->split = (int32_t*)(base + o);
  o = align_up(o + sizeof(int32_t) * (size_t)(G + 1));
  if (w) w->dx_router = base + o;
  o = align_up(o + b * T * dm);
  const int Gb = balance_splits(d->T);
  if (w) { w->bpart = (float*)(base + o); w->Gb = Gb; }
  o = align_up(o + sizeof(float) * (size_t)Gb * E);
  return o;
}

extern "C" {

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: outside this library's limits";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
  }
  return "unknown moe_status";
}

moe_status moe_workspace_size(const moe_desc* desc, int for_backward,
                              size_t* bytes) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_EINVAL;
  *bytes = for_backward ? bwd_ws_layout(desc, nullptr, nullptr)
                        : fwd_ws_layout(desc, nullptr, nullptr);
  return MOE_OK;
}

moe_status moe_router_workspace_size(const moe_desc* desc, size_t* bytes) {
  moe_status st = check_desc(desc);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_EINVAL;
  *bytes = router_ws_layout(desc, nullptr, nullptr);
  return MOE_OK;
}

moe_status moe_load_balance_stats(const moe_desc* d, const float* logits,
                                  const int32_t* counts, float* f,
                                  float* p_mean, float* aux, void* ws,
                                  size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!logits || !counts || !f || !p_mean || !aux || !ws) return MOE_EINVAL;
  if (ws_bytes < router_ws_layout(d, nullptr, nullptr)) return MOE_EWORKSPACE;
  RouterWs w;
  router_ws_layout(d, (char*)ws, &w);
  return hip_status(launch_balance_stats(logits, counts, d->T, d->E, d->gate,
                                         w.Gb, w.bpart, f, p_mean, aux,
                                         (hipStream_t)stream));
}

moe_status moe_update_route_bias(const moe_desc* d, const int32_t* counts,
                                 float* route_bias, float gamma, float target,
                                 int32_t rule, float* load, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!counts || !route_bias) return MOE_EINVAL;
  if (rule != 0 && rule != 1) return MOE_EINVAL;
  if (!(gamma == gamma) || !(target == target)) return MOE_EINVAL;
  if (d->T == 0) return MOE_OK;  // no load to balance: nothing is accessed
  return hip_status(launch_bias_update(counts, d->E, gamma, target, rule,
                                       route_bias, load, (hipStream_t)stream));
}

moe_status moe_balance_monitor(const moe_desc* d, const float* load_hist,
                               int32_t W, float* out, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (!load_hist || !out || W < 1) return MOE_EINVAL;
  return hip_status(launch_balance_monitor(load_hist, W, d->E, out,
                                           (hipStream_t)stream));
}

moe_status moe_quantize_mxfp8_t(const void* src, int64_t batch, int64_t rows,
                                int64_t cols, uint8_t* q, uint8_t* scales,
                                int64_t ldq, int64_t col_off, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0 || ldq < 0 || col_off < 0)
    return MOE_EINVAL;
  if (batch == 0 || rows == 0 || cols == 0) return MOE_OK;
  if (!src || !q || !scale_ptr_ok(scales) || col_off + rows > ldq)
    return MOE_EINVAL;
  if (rows % 32 || cols % 64 || ldq % 128 || col_off % 128 || rows > INT_MAX ||
      cols > INT_MAX || batch > 65535 || rows / 32 > 65535)
    return MOE_EUNSUPPORTED;
  return hip_status(launch_quantize_mxfp8_cols(src, batch, (int)rows,
                                               (int)cols, q + col_off, ldq,
                                               scales + col_off / 128 * batch * cols * 4,
                                               (hipStream_t)stream));
}

moe_status moe_router_backward(const moe_desc* d, const void* x,
                               const void* w_router, const float* logits,
                               const int32_t* topk_idx, const float* topk_w,
                               const float* d_topk_w, const int32_t* counts,
                               float aux_coef, float* d_logits,
                               void* d_w_router, void* dx, void* ws,
                               size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!x || !w_router || !logits || !topk_idx || !topk_w || !d_topk_w ||
      !d_logits || !d_w_router || !dx || !ws)
    return MOE_EINVAL;
  if (!(aux_coef == aux_coef) || (aux_coef != 0.0f && !counts))
    return MOE_EINVAL;
  if (ws_bytes < router_ws_layout(d, nullptr, nullptr)) return MOE_EWORKSPACE;
  RouterWs w;
  router_ws_layout(d, (char*)ws, &w);
  hipStream_t s = (hipStream_t)stream;
  const int dt = d->act_dtype, T = d->T, E = d->E, dm = d->d_model;
  hipError_t e;
#define MOE_TRY(x)                         \
  do {                                     \
    e = (x);                               \
    if (e != hipSuccess) return MOE_EHIP;  \
  } while (0)
  MOE_TRY(launch_router_grad(dt, logits, topk_idx, topk_w, d_topk_w,
                             aux_coef != 0.0f ? counts : nullptr, aux_coef, T,
                             E, d->K, d->gate, d_logits, w.dl_a, w.ld_dl, w.G,
                             w.split, s));
  // bf16 products on MFMA; fp32 (or shapes the tiles do not take) on SIMT
  const bool mfma = dt == MOE_BF16 && !force_simt();
  {  // the router's share of dx: d_logits Wr, added to dx
    GemmParams p = gp();
    p.M = T; p.N = dm; p.K = E;
    p.A = w.dl_a; p.lda = w.ld_dl;
    p.B = w_router; p.ldb = dm;
    p.C = dx; p.ldc = dm;
    if (mfma && mfma_supported(kOpRouterDx, p)) {
      MOE_TRY(gemm_mfma(kOpRouterDx, p, nullptr, s));  // accumulates into dx
    } else {
      p.C = w.dx_router;
      MOE_TRY(run_gemm(kOpRouterDx, dt, p, nullptr, s));
      MOE_TRY(launch_add_inplace(dt, dx, w.dx_router, (long)T * dm, s));
    }
  }
  {  // d Wr = d_logits^T x: partial sums over G token ranges, then their sum
    GemmParams p = gp();
    p.M = E; p.N = dm; p.G = w.G; p.off = w.split;
    p.A = w.dl_a; p.lda = w.ld_dl;
    p.B = x; p.ldb = dm;
    p.C = w.part; p.ldc = dm; p.sC = (long)E * dm;
    if (mfma && mfma_supported(kOpRouterDw, p))
      MOE_TRY(gemm_mfma(kOpRouterDw, p, nullptr, s));
    else
      MOE_TRY(run_gemm(kOpRouterDw, dt, p, nullptr, s));
    MOE_TRY(launch_reduce_parts(dt, w.part, (long)E * dm, w.G, d_w_router, s));
  }
#undef MOE_TRY
  return MOE_OK;
}

moe_status moe_route(const moe_desc* d, const void* x, const void* w_router,
                     const float* route_bias, const float* logits_in,
                     float* logits_out, int32_t* topk_idx, float* topk_w,
                     void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!topk_idx || !topk_w) return MOE_EINVAL;
  if (!logits_in && (!x || !w_router || !logits_out)) return MOE_EINVAL;
  return hip_status(do_route(d, x, w_router, route_bias, logits_in,
                             logits_out, topk_idx, topk_w,
                             (hipStream_t)stream));
}

moe_status moe_permute(const moe_desc* d, const void* x,
                       const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_src, int32_t* dest,
                       void* x_perm, uint8_t* x_perm_scales, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!x || !topk_idx || !counts || !offsets || !sorted_src || !dest ||
      !x_perm || !ws)
    return MOE_EINVAL;
  if (d->gemm_dtype == MOE_MXFP8 && !scale_ptr_ok(x_perm_scales))
    return MOE_EINVAL;
  if (ws_bytes < fwd_ws_layout(d, nullptr, nullptr)) return MOE_EWORKSPACE;
  FwdWs w;
  fwd_ws_layout(d, (char*)ws, &w);
  return hip_status(do_permute(d, x, topk_idx, counts, offsets, sorted_src,
                               dest, x_perm, x_perm_scales, w,
                               (hipStream_t)stream));
}

moe_status moe_grouped_gemm_swiglu(const moe_desc* d, const void* x_perm,
                                   const uint8_t* x_perm_scales,
                                   const int32_t* offsets,
                                   const moe_expert_weights* routed,
                                   const void* x_shared,
                                   const moe_expert_weights* shared, void* h,
                                   void* y_perm, void* y_shared, void* act_a,
                                   void* act_b, void* ws, size_t ws_bytes,
                                   void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!x_perm || !offsets || !weights_ok(routed) || !h || !y_perm || !ws)
    return MOE_EINVAL;
  const bool mx = d->gemm_dtype == MOE_MXFP8;
  if (mx && (!scale_ptr_ok(x_perm_scales) || !scale_ptr_ok(h) ||
             !mx_weights_ok(routed)))
    return MOE_EINVAL;
  const bool use_shared = x_shared && d->d_ff_shared > 0;
  if (use_shared && (!weights_ok(shared) || !y_shared)) return MOE_EINVAL;
  if ((d->flags & MOE_FLAG_SAVE_ACTS) && (!act_a || !act_b)) return MOE_EINVAL;
  if (ws_bytes < fwd_ws_layout(d, nullptr, nullptr)) return MOE_EWORKSPACE;
  FwdWs w;
  fwd_ws_layout(d, (char*)ws, &w);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_tile_prefix(offsets, d->E, w.tile_off, s);
  if (e != hipSuccess) return MOE_EHIP;
  if (mx) {
    if (use_shared && !mx_weights_ok(shared)) return MOE_EINVAL;
    return hip_status(do_experts_mx(d, x_perm, x_perm_scales, offsets, routed,
                                    use_shared ? x_shared : nullptr, shared, h,
                                    y_perm, y_shared, w, s, nullptr));
  }
  const bool save = d->flags & MOE_FLAG_SAVE_ACTS;
  return hip_status(do_experts(d, x_perm, offsets, routed,
                               use_shared ? x_shared : nullptr, shared, h,
                               y_perm, y_shared, save ? act_a : nullptr,
                               save ? act_b : nullptr, w, s, nullptr));
}

moe_status moe_unpermute_combine(const moe_desc* d, const void* y_perm,
                                 const int32_t* dest, const float* topk_w,
                                 const void* y_shared, void* out,
                                 void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!y_perm || !dest || !topk_w || !out) return MOE_EINVAL;
  return hip_status(launch_combine(d->act_dtype, y_perm, dest, topk_w,
                                   y_shared, out, d->T, d->K, d->d_model,
                                   (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Arguments of the whole forward (everything but the workspace).
moe_status check_fwd_args(const moe_desc* d, const moe_fwd_args* a) {
  if (!a || !a->x || !a->out || !weights_ok(&a->routed)) return MOE_EINVAL;
  if (!a->logits_in && (!a->w_router || !a->logits)) return MOE_EINVAL;
  if (!a->topk_idx || !a->topk_w || !a->counts || !a->offsets ||
      !a->sorted_src || !a->dest || !a->h || !a->y_perm)
    return MOE_EINVAL;
  // no x_perm: GEMM 1 gathers its rows from x (direct-to-LDS kernel only)
  const bool gather = a->x_perm == nullptr;
  if (gather && (d->act_dtype != MOE_BF16 || force_simt() ||
                 !gemm1_gather_supported(d->d_model) ||
                 (long)d->T * d->d_model * 2 >= (1L << 31)))
    return MOE_EUNSUPPORTED;
  const bool shared = d->d_ff_shared > 0;
  if (shared && (!weights_ok(&a->shared) || !a->y_shared)) return MOE_EINVAL;
  const bool save = d->flags & MOE_FLAG_SAVE_ACTS;
  if (save && (!a->act_a || !a->act_b)) return MOE_EINVAL;
  const bool mx = d->gemm_dtype == MOE_MXFP8;
  if (mx && ((!gather && !scale_ptr_ok(a->x_perm_scales)) ||
             !scale_ptr_ok(a->h) || !mx_weights_ok(&a->routed)))
    return MOE_EINVAL;
  if (mx && shared && !mx_weights_ok(&a->shared)) return MOE_EINVAL;
  return MOE_OK;
}

// The whole forward in a validated workspace of the required size.
moe_status forward_in(const moe_desc* d, const moe_fwd_args* a, void* ws,
                      hipStream_t s) {
  const bool gather = a->x_perm == nullptr;
  const bool shared = d->d_ff_shared > 0;
  const bool save = d->flags & MOE_FLAG_SAVE_ACTS;
  const bool mx = d->gemm_dtype == MOE_MXFP8;
  FwdWs w;
  fwd_ws_layout(d, (char*)ws, &w);
  record(a->events[0], s);
  bool ranked = false;
  hipError_t e = do_route(d, a->x, a->w_router, a->route_bias, a->logits_in,
                          a->logits, a->topk_idx, a->topk_w, s, &w, &ranked);
  if (e != hipSuccess) return MOE_EHIP;
  record(a->events[1], s);
  e = do_permute(d, a->x, a->topk_idx, a->counts, a->offsets, a->sorted_src,
                 a->dest, a->x_perm, a->x_perm_scales, w, s, ranked);
  if (e != hipSuccess) return MOE_EHIP;
  record(a->events[2], s);
  const int32_t* gsrc = gather ? a->sorted_src : nullptr;
  if (mx)
    e = do_experts_mx(d, a->x_perm, a->x_perm_scales, a->offsets, &a->routed,
                      shared ? a->x : nullptr, &a->shared, a->h, a->y_perm,
                      a->y_shared, w, s, a->events[3], gsrc,
                      save ? a->act_a : nullptr, save ? a->act_b : nullptr);
  else
    e = do_experts(d, gather ? a->x : a->x_perm, a->offsets, &a->routed,
                   shared ? a->x : nullptr, &a->shared, a->h, a->y_perm,
                   a->y_shared, save ? a->act_a : nullptr,
                   save ? a->act_b : nullptr, w, s, a->events[3], gsrc);
  if (e != hipSuccess) return MOE_EHIP;
  record(a->events[4], s);
  e = launch_combine(d->act_dtype, a->y_perm, a->dest, a->topk_w,
                     shared ? a->y_shared : nullptr, a->out, d->T, d->K,
                     d->d_model, s);
  if (e != hipSuccess) return MOE_EHIP;
  record(a->events[5], s);
  return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Static device scratch of the allocation-free forward. In host code the
// name `scratch` is only a stand-in for the symbol: its device address (one
// per GPU) comes from hipGetSymbolAddress with that GPU current, and only
// that address is handed to kernels.
static __device__ __align__(256) char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per GPU

// This GPU's copy of the scratch (looked up on the first call on each
// device, with that device current); nullptr if HIP cannot provide it.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();  // leave no sticky error for the next call
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

moe_status moe_forward(const moe_desc* d, const moe_fwd_args* a, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!ws) return MOE_EINVAL;
  st = check_fwd_args(d, a);
  if (st != MOE_OK) return st;
  if (ws_bytes < fwd_ws_layout(d, nullptr, nullptr)) return MOE_EWORKSPACE;
  return forward_in(d, a, ws, (hipStream_t)stream);
}

moe_status moe_forward_noalloc(const moe_desc* d, const moe_fwd_args* a,
                               void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  st = check_fwd_args(d, a);
  if (st != MOE_OK) return st;
  if (fwd_ws_layout(d, nullptr, nullptr) > MOE_STATIC_SCRATCH_BYTES)
    return MOE_EUNSUPPORTED;
  void* ws = device_scratch();
  if (!ws) return MOE_EHIP;
  return forward_in(d, a, ws, (hipStream_t)stream);
}

moe_status moe_backward(const moe_desc* d, const moe_bwd_args* a, void* ws,
                        size_t ws_bytes, void* stream) {
  moe_status st = check_desc(d);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;  // nothing is accessed
  if (!a || !ws || !a->dy || !weights_ok(&a->routed) || !a->topk_w ||
      !a->offsets || !a->dest || !a->x_perm || !a->h || !a->y_perm ||
      !a->dx || !a->dw1 || !a->dw3 || !a->dw2 || !a->d_topk_w)
    return MOE_EINVAL;
  if ((a->act_a == nullptr) != (a->act_b == nullptr)) return MOE_EINVAL;
  if (d->gemm_dtype == MOE_MXFP8) {
    if (!scale_ptr_ok(a->x_perm_scales) || !scale_ptr_ok(a->h) || !a->w2t ||
        !scale_ptr_ok(a->w2t_scales) || !a->w13t ||
        !scale_ptr_ok(a->w13t_scales) || !mx_weights_ok(&a->routed))
      return MOE_EINVAL;
    if (d->d_ff_shared > 0 &&
        (!mx_weights_ok(&a->shared) || !a->dws1 || !a->dws3 || !a->dws2 ||
         !a->ws2t || !scale_ptr_ok(a->ws2t_scales) || !a->ws13t ||
         !scale_ptr_ok(a->ws13t_scales)))
      return MOE_EINVAL;
    if (ws_bytes < bwd_ws_layout(d, nullptr, nullptr)) return MOE_EWORKSPACE;
    return hip_status(do_backward_mx(d, a, ws, (hipStream_t)stream));
  }
  const bool shared = d->d_ff_shared > 0;
  if (shared && (!weights_ok(&a->shared) || !a->dws1 || !a->dws3 || !a->dws2))
    return MOE_EINVAL;
  if (ws_bytes < bwd_ws_layout(d, nullptr, nullptr)) return MOE_EWORKSPACE;
  BwdWs w;
  bwd_ws_layout(d, (char*)ws, &w);
  hipStream_t s = (hipStream_t)stream;
  const int TK = d->T * d->K, dm = d->d_model, f = d->d_ff, E = d->E;
  const int dt = d->act_dtype;
  hipError_t e;
#define MOE_TRY(x)                         \
  do {                                     \
    e = (x);                               \
    if (e != hipSuccess) return MOE_EHIP;  \
  } while (0)
  record(a->events[0], s);
  MOE_TRY(launch_tile_prefix(a->offsets, E, w.tile_off, s));
  // combine^T: dy_perm = w * dy, d_topk_w = <dy, y_perm>
  MOE_TRY(launch_combine_bwd(dt, a->dy, a->y_perm, a->dest, a->topk_w,
                             w.dy_perm, a->d_topk_w, d->T, d->K, dm, s));
  record(a->events[1], s);
  // pre-activations: saved, or recomputed into the da/db buffers
  const void* sa = a->act_a;
  const void* sb = a->act_b;
  if (!sa) {
    MOE_TRY(do_gemm1(d, a->x_perm, a->offsets, TK, E, a->routed.w1,
                     a->routed.w3, f, nullptr, w.da, w.db, w.tile_off, s));
    sa = w.da;
    sb = w.db;
  }
  const int fs = d->d_ff_shared;
  if (shared) {  // shared expert over every token: h, a, b
    MOE_TRY(launch_split(d->T, 1, w.srange, s));
    MOE_TRY(do_gemm1(d, a->x, nullptr, d->T, 1, a->shared.w1, a->shared.w3,
                     fs, w.sh, w.sa, w.sb, w.tile_off, s));
  }
  record(a->events[2], s);
  {  // dh = dy_perm W2_e, then (da, db) from the SwiGLU derivative
    GemmParams p = gp();
    p.M = TK; p.N = f; p.K = dm; p.G = E; p.off = a->offsets;
    p.A = w.dy_perm; p.lda = dm;
    p.B = a->routed.w2; p.ldb = f; p.sB = (long)dm * f;
    p.C = w.da; p.C2 = w.db; p.ldc = f;
    p.aux_a = sa; p.aux_b = sb;
    MOE_TRY(run_gemm(kOpDgrad2, dt, p, w.tile_off, s));
  }
  if (shared) {  // ungated: dh_s = dy Ws2, (da_s, db_s) in place of (a_s, b_s)
    GemmParams p = gp();
    p.M = d->T; p.N = fs; p.K = dm;
    p.A = a->dy; p.lda = dm;
    p.B = a->shared.w2; p.ldb = fs;
    p.C = w.sa; p.C2 = w.sb; p.ldc = fs;
    p.aux_a = w.sa; p.aux_b = w.sb;
    MOE_TRY(run_gemm(kOpDgrad2, dt, p, w.tile_off, s));
  }
  record(a->events[3], s);
  {  // dx_perm = da W1_e + db W3_e
    GemmParams p = gp();
    p.M = TK; p.N = dm; p.K = 2 * f; p.K1 = f; p.G = E; p.off = a->offsets;
    p.A = w.da; p.A2 = w.db; p.lda = f;
    p.B = a->routed.w1; p.B2 = a->routed.w3; p.ldb = dm; p.sB = (long)f * dm;
    p.C = w.dx_perm; p.ldc = dm;
    p.slots = d->flags & MOE_FLAG_NO_TAIL_SPLIT ? 0 : -1;
    MOE_TRY(run_gemm(kOpDgrad1, dt, p, w.tile_off, s));
  }
  if (shared) {  // dx_s = da_s Ws1 + db_s Ws3
    GemmParams p = gp();
    p.M = d->T; p.N = dm; p.K = 2 * fs; p.K1 = fs;
    p.A = w.sa; p.A2 = w.sb; p.lda = fs;
    p.B = a->shared.w1; p.B2 = a->shared.w3; p.ldb = dm;
    p.C = w.sdx; p.ldc = dm;
    MOE_TRY(run_gemm(kOpDgrad1, dt, p, w.tile_off, s));
  }
  record(a->events[4], s);
  MOE_TRY(launch_combine(dt, w.dx_perm, a->dest, nullptr,
                         shared ? w.sdx : nullptr, a->dx, d->T, d->K, dm, s));
  record(a->events[5], s);
  {  // dW2_e = dy_perm_e^T h_e
    GemmParams p = gp();
    p.M = dm; p.N = f; p.G = E; p.off = a->offsets; p.k_total = TK;
    p.A = w.dy_perm; p.lda = dm;
    p.B = a->h; p.ldb = f;
    p.C = a->dw2; p.ldc = f; p.sC = (long)dm * f;
    MOE_TRY(run_gemm(kOpWgrad, dt, p, w.tile_off, s));
  }
  if (shared) {  // dWs2 = dy^T h_s
    GemmParams p = gp();
    p.M = dm; p.N = fs; p.G = 1; p.off = w.srange; p.k_total = d->T;
    p.A = a->dy; p.lda = dm;
    p.B = w.sh; p.ldb = fs;
    p.C = a->dws2; p.ldc = fs;
    MOE_TRY(run_gemm(kOpWgrad, dt, p, w.tile_off, s));
  }
  record(a->events[6], s);
  for (int which = 0; which < 2; ++which) {  // dW1_e = da^T x_perm, dW3_e
    GemmParams p = gp();
    p.M = f; p.N = dm; p.G = E; p.off = a->offsets; p.k_total = TK;
    p.A = which ? w.db : w.da; p.lda = f;
    p.B = a->x_perm; p.ldb = dm;
    p.C = which ? a->dw3 : a->dw1; p.ldc = dm; p.sC = (long)f * dm;
    MOE_TRY(run_gemm(kOpWgrad, dt, p, w.tile_off, s));
    if (shared) {  // dWs1 = da_s^T x, dWs3 = db_s^T x
      GemmParams q = gp();
      q.M = fs; q.N = dm; q.G = 1; q.off = w.srange; q.k_total = d->T;
      q.A = which ? w.sb : w.sa; q.lda = fs;
      q.B = a->x; q.ldb = dm;
      q.C = which ? a->dws3 : a->dws1; q.ldc = dm;
      MOE_TRY(run_gemm(kOpWgrad, dt, q, w.tile_off, s));
    }
  }
  record(a->events[7], s);
#undef MOE_TRY
  return MOE_OK;
}

moe_status moe_quantize_mxfp8(const void* src_bf16, int64_t rows,
                              int64_t cols, uint8_t* q, uint8_t* scales,
                              void* stream) {
  if (!src_bf16 || !q || !scale_ptr_ok(scales) || rows < 0 || cols <= 0)
    return MOE_EINVAL;
  if (cols % 128) return MOE_EUNSUPPORTED;
  if (rows == 0) return MOE_OK;
  return hip_status(launch_quantize_mxfp8(src_bf16, rows, cols, q, scales,
                                          (hipStream_t)stream));
}

}  // extern "C"
