/*
 * moe.h - C ABI of a dropless Mixture-of-Experts expert layer for one AMD
 * Instinct MI355X (gfx950): router, top-K gating, expert histogram and
 * stable permutation, ragged grouped SwiGLU GEMMs on MFMA, gate-weighted
 * combine, optional shared expert, backward pass, and an MXFP8 forward.
 *
 * Pages cited:
 *   [P1] kongchang.com, "JAX中加速Dropless MoE训练：NVIDIA Transformer
 *        Engine解析", section "Dropless MoE：解决 token 丢弃问题" (every token
 *        copy reaches its experts; no capacity, no drops) and section
 *        "高效的分组矩阵运算" (grouped GEMM over ragged groups, no padding).
 *   [P2] ai.warp-studio.com, "JAXにおけるDropless MoE訓練をNVIDIA Transformer
 *        Engineで劇的に加速する技術分析", section on the TE mechanisms
 *        (grouped GEMM in one call over ragged experts; group-aware MXFP8;
 *        shapes that stay on the device so graphs need no host shapes).
 *   [P3] quant67.com, "【大模型基础设施工程】08：MoE 训练工程": §4.1 softmax
 *        top-K gate with renormalisation, §4.3 sigmoid gate, §5 shared
 *        expert, §6.3 route bias for selection only, §9 the single-GPU
 *        MoE layer (SwiGLU experts, per-expert gather, index_add combine,
 *        load counts), §11.3 sparse backward, §12.5 sort-based permutation
 *        and its inverse, §12.7 gate math in fp32, §13.6 fp8 with per-tile
 *        scales and fp32 accumulation.
 *
 * Conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer, row-major, 16-byte aligned,
 *     owned by the caller. The library allocates nothing, frees nothing,
 *     never synchronises, and keeps no state between calls (reentrant).
 *   - Weights use the linear-layer [out, in] layout: W1, W3 are
 *     [E, d_ff, d_model], W2 is [E, d_model, d_ff], the router is
 *     [E, d_model]; shared-expert weights are [d_ff_shared, d_model] and
 *     [d_model, d_ff_shared].
 *   - "act" dtype (desc->act_dtype) is the element type of x, weights,
 *     x_perm, h, y_perm, y_shared, out and gradients: fp32 or bf16.
 *     Logits, gate weights and all accumulation are fp32.
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is
 *     enqueued asynchronously; nothing depends on host-visible shapes, so
 *     every call can be captured in a HIP graph and replayed with new
 *     routing.
 *   - Errors: only host-checkable arguments are validated. On any error
 *     no work is enqueued and a status != MOE_OK is returned. MOE_EHIP
 *     reports a launch error from the HIP runtime. Device-side data (e.g.
 *     an expert id outside [0, E) in topk_idx) is not validated.
 *   - T == 0 is valid: the descriptor is checked, then MOE_OK is returned
 *     with nothing enqueued and no pointer read (pointers may be NULL).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK            0
#define MOE_EINVAL        1  /* NULL pointer, negative or inconsistent size */
#define MOE_EUNSUPPORTED  2  /* valid but outside this library's limits   */
#define MOE_EWORKSPACE    3  /* workspace smaller than moe_workspace_size */
#define MOE_EHIP          4  /* HIP runtime reported an error             */

/* element types */
#define MOE_F32    0
#define MOE_BF16   1
#define MOE_MXFP8  2  /* gemm_dtype only: E4M3 elements, E8M0 scale per 32 */

/* gating */
#define MOE_GATE_SOFTMAX 0  /* [P3 §4.1] */
#define MOE_GATE_SIGMOID 1  /* [P3 §4.3] */

/* flags */
#define MOE_FLAG_SAVE_ACTS 1  /* forward stores the pre-activations a, b */
/* The bf16 expert GEMMs run a partial last round of 256-row tiles (at most
   a quarter of the CUs' worth of tiles) as 128 x 128 quarter tiles by
   default; this flag keeps every tile at full size. Results are
   bit-identical either way (same accumulation order per output). */
#define MOE_FLAG_NO_TAIL_SPLIT 2

/* limits of this library */
#define MOE_K_MAX 16
#define MOE_E_MAX 1024
/* size of the static device scratch moe_forward_noalloc works in */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)

/* Number of stage-boundary events moe_forward / moe_backward can record. */
#define MOE_FWD_NEVENTS 6
#define MOE_BWD_NEVENTS 8

typedef struct moe_desc {
  int32_t T;            /* tokens (batch x sequence flattened), >= 0       */
  int32_t d_model;      /* multiple of 8 (bf16/fp32), of 128 (MXFP8)       */
  int32_t d_ff;         /* routed expert hidden size, same rule            */
  int32_t E;            /* routed experts, 1..MOE_E_MAX                    */
  int32_t K;            /* experts per token, 1..min(E, MOE_K_MAX)         */
  int32_t d_ff_shared;  /* shared expert hidden size, 0 = none [P3 §5]     */
  int32_t gate;         /* MOE_GATE_SOFTMAX | MOE_GATE_SIGMOID             */
  int32_t act_dtype;    /* MOE_F32 | MOE_BF16                              */
  int32_t gemm_dtype;   /* = act_dtype, or MOE_MXFP8 (bf16 act; d_model,
                           d_ff and d_ff_shared multiples of 128)         */
  int32_t flags;        /* MOE_FLAG_*                                      */
} moe_desc;

/* MX scale layout. Every MXFP8 operand here is E4M3 codes [rows, cols]
 * (cols a multiple of 128) with one E8M0 code per 32 consecutive elements
 * of a row, rows * cols / 32 bytes grouped by 128-column span: the code of
 * block b (columns 32 b .. 32 b + 31) of row r is at byte
 *     ((b / 4) * rows + r) * 4 + b % 4,
 * i.e. [cols / 128][rows][4]. One span's four codes of a row form one
 * aligned 4-byte word, and the words of consecutive rows are adjacent, so
 * the scales that a 128-wide k-tile of a GEMM needs for 32 consecutive
 * rows are one 128-byte line (a row-major [rows][cols / 32] array would
 * spread them over 32 lines). A batch of operands ([B, rows, cols]) is laid
 * out as the one operand of B * rows rows that stacks them. The block rule
 * itself is moe_quantize_mxfp8's.
 * Scale arrays (and an MXFP8 h buffer, which ends in one) start on a
 * 4-byte boundary; calls given another return MOE_EINVAL. */

/* One set of SwiGLU expert weights [P3 §9]: y = W2 (silu(W1 x) * (W3 x)).
 * For the routed experts the leading dimension is E; for the shared
 * expert it is absent. With gemm_dtype == MOE_MXFP8 the w* pointers hold
 * E4M3 bytes (quantised by moe_quantize_mxfp8) and *_scales hold the
 * E8M0 codes, one per 32 elements along the row, in the MX scale layout
 * of the stacked matrices: w1/w3 scales of E*d_ff rows and d_model
 * columns, w2 scales of E*d_model rows and d_ff columns. */
typedef struct moe_expert_weights {
  const void* w1;
  const void* w3;
  const void* w2;
  const uint8_t* w1_scales;
  const uint8_t* w3_scales;
  const uint8_t* w2_scales;
} moe_expert_weights;

/* Forward arguments. Required unless marked optional. */
typedef struct moe_fwd_args {
  const void* x;              /* [T, d_model] act                            */
  const void* w_router;       /* [E, d_model] act; unused if logits_in       */
  const float* route_bias;    /* optional [E]: selection only [P3 §6.3]      */
  const float* logits_in;     /* optional [T, E]: bypasses the router GEMM   */
  moe_expert_weights routed;  /* [E, ...]                                    */
  moe_expert_weights shared;  /* used iff d_ff_shared > 0                    */
  void* out;                  /* [T, d_model] act                            */
  /* routing state, kept for backward */
  float* logits;              /* [T, E] fp32; required iff logits_in == NULL */
  int32_t* topk_idx;          /* [T, K] expert ids, rank order               */
  float* topk_w;              /* [T, K] renormalised gate weights            */
  int32_t* counts;            /* [E] copies per expert                       */
  int32_t* offsets;           /* [E+1] exclusive prefix of counts            */
  int32_t* sorted_src;        /* [T*K] copy j = t*K+k at each sorted slot    */
  int32_t* dest;              /* [T*K] sorted slot of each copy j            */
  /* activations */
  void* x_perm;               /* [T*K, d_model] act (MXFP8: E4M3 bytes), or
                                 NULL: then GEMM 1 reads row p straight from
                                 x[sorted_src[p] / K] (MXFP8: from x
                                 quantised once in the workspace) and the
                                 permute writes only the indices. NULL
                                 needs bf16 act, d_model % 64 == 0 and
                                 T * d_model * 2 < 2^31, else
                                 MOE_EUNSUPPORTED. moe_backward still needs
                                 a materialised x_perm.                     */
  uint8_t* x_perm_scales;     /* MXFP8 with x_perm: E8M0, MX scale layout of
                                 T*K rows, d_model columns                  */
  void* h;                    /* [T*K, d_ff] act. MXFP8: E4M3 codes [T*K,
                                 d_ff] then their E8M0 scales (MX scale
                                 layout, T*K * d_ff / 32 bytes; fits in a
                                 bf16-sized buffer)                         */
  void* y_perm;               /* [T*K, d_model] act, unweighted expert out   */
  void* y_shared;             /* [T, d_model] act; required iff shared       */
  void* act_a;                /* [T*K, d_ff] act; required iff SAVE_ACTS     */
  void* act_b;                /* [T*K, d_ff] act; required iff SAVE_ACTS     */
  void* events[MOE_FWD_NEVENTS]; /* optional hipEvent_t, recorded at: start,
                                    after routing, after permute, after GEMM1,
                                    after GEMM2 (+shared), after combine      */
} moe_fwd_args;

/* Backward arguments: gradients of sum(dy * out) with the routing fixed
 * and the gate weights as leaves [P3 §11.3]. Experts that received no
 * token get dW = 0. */
typedef struct moe_bwd_args {
  const void* dy;             /* [T, d_model] act                            */
  const void* x;              /* [T, d_model] act                            */
  moe_expert_weights routed;  /* act dtype (MXFP8: the forward's MX weights)  */
  moe_expert_weights shared;
  /* saved forward state (as written by moe_forward) */
  const int32_t* topk_idx;
  const float* topk_w;
  const int32_t* offsets;
  const int32_t* sorted_src;
  const int32_t* dest;
  const void* x_perm;
  const void* h;
  const void* y_perm;
  const void* act_a;          /* optional: NULL = recompute a, b             */
  const void* act_b;
  /* outputs */
  void* dx;                   /* [T, d_model] act                            */
  void* dw1;                  /* [E, d_ff, d_model] act                      */
  void* dw3;                  /* [E, d_ff, d_model] act                      */
  void* dw2;                  /* [E, d_model, d_ff] act                      */
  float* d_topk_w;            /* [T, K] fp32                                 */
  void* dws1;                 /* [d_ff_shared, d_model] act; iff shared      */
  void* dws3;                 /* [d_ff_shared, d_model] act; iff shared      */
  void* dws2;                 /* [d_model, d_ff_shared] act; iff shared      */
  /* MXFP8 backward only (gemm_dtype MOE_MXFP8): the forward's MX state and
     the weights quantised for the transposed products (moe_quantize_mxfp8_t):
     x_perm and h then hold the forward's E4M3 codes (h: codes then scales),
     routed the forward's MX weights (for the recomputed a, b). */
  const uint8_t* x_perm_scales; /* E8M0, MX scale layout (as the forward's)  */
  const uint8_t* w2t;         /* [E, d_ff, d_model] E4M3: W2^T, blocks along
                                 d_model                                    */
  const uint8_t* w2t_scales;  /* E*d_ff rows, d_model columns (stacked)     */
  const uint8_t* w13t;        /* [E, d_model, 2*d_ff] E4M3: [W1^T | W3^T],
                                 blocks along d_ff                          */
  const uint8_t* w13t_scales; /* E*d_model rows, 2*d_ff columns (stacked)   */
  /* the same for the shared expert (MXFP8 with d_ff_shared > 0): shared
     holds its forward MX weights; ws2t [d_ff_shared, d_model],
     ws13t [d_model, 2*d_ff_shared], as w2t and w13t with E = 1 */
  const uint8_t* ws2t;
  const uint8_t* ws2t_scales;
  const uint8_t* ws13t;
  const uint8_t* ws13t_scales;
  void* events[MOE_BWD_NEVENTS]; /* optional hipEvent_t stage boundaries     */
} moe_bwd_args;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_str(moe_status s);

/* Bytes of scratch workspace moe_permute / moe_grouped_gemm_swiglu /
 * moe_forward (for_backward == 0) or moe_backward (for_backward != 0)
 * need for this descriptor. Written to *bytes. */
moe_status moe_workspace_size(const moe_desc* desc, int for_backward,
                              size_t* bytes);

/* Router and gate [P3 §4.1, §4.3, §6.3, §12.7].
 * logits = x W_router^T (fp32 accumulate) unless logits_in is given.
 * Selection key: logit (+ route_bias[e] if given, added in fp32); -0.0
 * equals +0.0 and NaN counts as -inf. The K experts with the largest
 * keys are chosen, ties to the lowest expert id, and written to
 * topk_idx[t, 0..K-1] in (key descending, id ascending) order.
 * Weights use the raw logits: softmax over the K selected logits, or
 * sigmoid(logit) / sum of the K sigmoids; they sum to 1 (1/K each if
 * the sum is 0). logits_out receives the logits when computed (may be
 * NULL if logits_in is given). */
moe_status moe_route(const moe_desc* desc, const void* x,
                     const void* w_router, const float* route_bias,
                     const float* logits_in, float* logits_out,
                     int32_t* topk_idx, float* topk_w, void* stream);

/* Histogram, prefix scan and stable permutation [P3 §9, §12.5].
 * counts[e] = #{(t,k): topk_idx[t,k] == e}; offsets = exclusive prefix
 * (offsets[E] = T*K: nothing dropped, nothing padded [P1]). Copies are
 * ordered by (expert, j = t*K+k): sorted_src[p] = j, dest[j] = p, and
 * x_perm[p] = x[j / K] (bit copy; with gemm_dtype MXFP8, E4M3 codes plus
 * E8M0 scales in x_perm_scales). Integer work, bit-exact, atomic-free on
 * global memory. */
moe_status moe_permute(const moe_desc* desc, const void* x,
                       const int32_t* topk_idx, int32_t* counts,
                       int32_t* offsets, int32_t* sorted_src, int32_t* dest,
                       void* x_perm, uint8_t* x_perm_scales, void* ws,
                       size_t ws_bytes, void* stream);

/* Ragged grouped SwiGLU GEMMs [P1 grouped GEMM; P2; P3 §9 Expert]. For
 * each expert e and sorted rows p in [offsets[e], offsets[e+1]):
 *   a = x_perm[p] W1_e^T, b = x_perm[p] W3_e^T   (fp32 accumulate)
 *   h[p] = silu(a) * b                           (stored in act dtype)
 *   y_perm[p] = h[p] W2_e^T                      (stored in act dtype)
 * The tile list over (expert, row tile) is built on the device from
 * offsets; no host synchronisation. act_a/act_b (optional) receive a, b.
 * MXFP8 (gemm_dtype): both operands of both GEMMs are E4M3 with one E8M0
 * scale per 32 elements along the contraction dimension (x_perm and W1/W3
 * along d_model, h and W2 along d_ff), accumulated in fp32 [P2 MXFP8
 * grouped GEMM; P3 §13.6 per-tile scales]; h is quantised from the fp32
 * SwiGLU value in the GEMM 1 epilogue and stored in the h buffer as codes
 * then scales; y_perm is bf16.
 * If x_shared is non-NULL and d_ff_shared > 0, the shared expert runs on
 * every token: y_shared = SwiGLU_shared(x_shared). MXFP8: x_perm and
 * x_perm_scales are E4M3/E8M0 and all weights (routed and shared) must be
 * quantised; x_shared stays bf16 and is quantised into the workspace. */
moe_status moe_grouped_gemm_swiglu(const moe_desc* desc, const void* x_perm,
                                   const uint8_t* x_perm_scales,
                                   const int32_t* offsets,
                                   const moe_expert_weights* routed,
                                   const void* x_shared,
                                   const moe_expert_weights* shared,
                                   void* h, void* y_perm, void* y_shared,
                                   void* act_a, void* act_b, void* ws,
                                   size_t ws_bytes, void* stream);

/* Gate-weighted unpermute and combine [P3 §9, §12.5 step 6, §5]:
 * out[t] = sum_{k<K} topk_w[t,k] * y_perm[dest[t*K+k]] (+ y_shared[t]),
 * accumulated in fp32 in k order and rounded once. Deterministic: each
 * output row is owned by one workgroup; no atomics. y_shared may be NULL. */
moe_status moe_unpermute_combine(const moe_desc* desc, const void* y_perm,
                                 const int32_t* dest, const float* topk_w,
                                 const void* y_shared, void* out,
                                 void* stream);

/* Whole forward of the layer [P3 §9, the MoE layer and its forward; §5
 * shared expert; P2 section on the TE mechanisms: routing, dispatch, the
 * grouped GEMM and the combine in one device-resident pass]: moe_route,
 * moe_permute, moe_grouped_gemm_swiglu (+ shared expert) and
 * moe_unpermute_combine in sequence on one stream, with the same argument
 * meanings (see moe_fwd_args). The caller owns every buffer in args and
 * the workspace (>= moe_workspace_size(desc, 0)). args->x_perm == NULL
 * (bf16 or MXFP8, d_model % 64 == 0, T * d_model * 2 < 2^31) selects the
 * gathered GEMM 1: the permute writes only the indices and GEMM 1 reads
 * its rows from x through sorted_src [P3 §9, its engineering notes on
 * grouped GEMMs over per-expert row groups]; otherwise MOE_EUNSUPPORTED.
 * Errors: NULL required pointers -> MOE_EINVAL; workspace too small ->
 * MOE_EWORKSPACE; nothing is enqueued on error. */
moe_status moe_forward(const moe_desc* desc, const moe_fwd_args* args,
                       void* ws, size_t ws_bytes, void* stream);

/* Allocation-free whole forward, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same computation, arguments and errors as
 * moe_forward, except that the workspace is not passed in: it is a static
 * device array of MOE_STATIC_SCRATCH_BYTES (64 MiB) that the library holds
 * on every GPU it runs on, from the first call there until the process
 * ends. The caller still owns every buffer in args. The call allocates and
 * frees nothing. The stream must belong to the current device.
 *   - MOE_EUNSUPPORTED when moe_workspace_size(desc, 0) exceeds
 *     MOE_STATIC_SCRATCH_BYTES (e.g. a shared expert's T x d_ff_shared
 *     hidden, or under MXFP8 the quantised x, beyond it);
 *   - MOE_EHIP when the device address of the array cannot be obtained;
 *   - otherwise as moe_forward.
 * Every call on one GPU works in that GPU's one array, which keeps the
 * previous call's contents (no part of it needs to start at zero: each
 * kernel writes what it later reads). Calls on one stream are ordered;
 * calls that overlap in time on one GPU (different streams, or different
 * host threads) race on the array and must not be made. */
moe_status moe_forward_noalloc(const moe_desc* desc, const moe_fwd_args* args,
                               void* stream);

/* Whole backward (see moe_bwd_args). Deterministic: weight gradients are
 * owned tile by tile (no split-K atomics). The shared expert [P3 §5] is an
 * ungated SwiGLU FFN over every token: its pre-activations are recomputed,
 * its gradients written to dws1/dws3/dws2 and its share of dx added into
 * dx.
 * MXFP8 descriptors [P3 §13.6]: the data-gradient products run on the
 * scaled MFMA with both operands MX-quantised along their contraction:
 *   dh = Q(dy_perm) . w2t  (dy_perm = w * dy in bf16, blocks along d_model)
 *   dx_perm = Q([da | db]) . w13t  (da, db in bf16, blocks along d_ff)
 * with a, b saved by the forward (MOE_FLAG_SAVE_ACTS: the MX GEMM 1 keeps
 * its fp32 accumulators in bf16) or else recomputed by it from x_perm;
 * the weight gradients are bf16 products of the operands the forward
 * multiplied: dW2 = dy_perm^T h, dW1 = da^T x_perm, dW3 = db^T x_perm with
 * h and x_perm dequantised from the forward's MX codes (exact in bf16).
 * Needs x_perm_scales, w2t, w13t and their scales and the routed MX
 * weights with scales. A shared expert runs the same way as one dense
 * group over every token (dy ungated; x and dy quantised into the
 * workspace; its a, b and MX h recomputed by the MX GEMM 1) and needs the
 * shared MX weights and ws2t, ws13t with their scales. */
moe_status moe_backward(const moe_desc* desc, const moe_bwd_args* args,
                        void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of moe_router_backward and of moe_load_balance_stats
 * (independent of their pointers). */
moe_status moe_router_workspace_size(const moe_desc* desc, size_t* bytes);

/* Router backward: the gate-weight gradient d_topk_w [T, K] (from
 * moe_backward) carried through the renormalised gate [P3 §4.1, §4.3] to
 * the logits, the router weights and the tokens. The selection is held
 * fixed (it is piecewise constant in the logits), so only the K selected
 * logits of a token get gradient:
 *   softmax: d_logits[t, e_k] = w_k (d_w_k - sum_j w_j d_w_j);
 *   sigmoid: d_logits[t, e_k] = s_k (1 - s_k) / S (d_w_k - sum_j w_j d_w_j),
 *            s = sigmoid(logit), S = sum of the selected s (0 if S == 0);
 * with w = topk_w and logits the forward's fp32 logits [T, E] (the raw
 * logits: a route bias only moves the selection).
 * With aux_coef != 0 the loss also holds aux_coef times the balance loss
 * of moe_load_balance_stats [P3 §6.2]; its gradient at fixed
 * f = counts / T (counts [E] from the forward, required then, ignored
 * otherwise) is added to every logit j of token t:
 *   aux_coef (E / T) q_tj (f_j - sum_i f_i P_ti),
 *   q = P (softmax), q_tj = s_tj (1 - s_tj) / sum_i s_ti (sigmoid),
 * with P the full-row gate probabilities defined there.
 * Writes d_logits [T, E] fp32 (zero off the selection when aux_coef == 0)
 * and d_w_router [E, d_model] = d_logits^T x in the activation dtype, and
 * ADDS d_logits * w_router [T, d_model] into dx (in/out, activation dtype:
 * e.g. moe_backward's dx, so that dx becomes the whole layer's input
 * gradient). x and w_router are as in the forward. d_w_router is the sum
 * of fixed token-range partial sums taken in a fixed order:
 * deterministic. MOE_EINVAL on a NULL pointer, a NaN aux_coef or a
 * nonzero aux_coef without counts; MOE_EWORKSPACE if
 * ws_bytes < moe_router_workspace_size. */
moe_status moe_router_backward(const moe_desc* desc, const void* x,
                               const void* w_router, const float* logits,
                               const int32_t* topk_idx, const float* topk_w,
                               const float* d_topk_w, const int32_t* counts,
                               float aux_coef, float* d_logits,
                               void* d_w_router, void* dx, void* ws,
                               size_t ws_bytes, void* stream);

/* Load-balance statistics of one routing [P3 §6.2, §9], from the
 * forward's fp32 logits [T, E] and counts [E]:
 *   f[e]      = counts[e] / T, the share of tokens whose top-K holds e
 *               (sums to K; the layer's load statistic counts / (T K) is
 *               f / K);
 *   p_mean[e] = (1 / T) sum_t P[t, e], the mean gate probability, with
 *               P[t, :] = softmax(logits[t, :]) over all E experts
 *               (softmax gate) or sigmoid(logits[t, :]) divided by its sum
 *               over all E (sigmoid gate, raw logits; 1/E each if every
 *               sigmoid of the row is zero in fp32);
 *   aux[0]    = E sum_e f[e] p_mean[e], the auxiliary balance loss before
 *               its coefficient (E scales it to 1 for top-1 routing that
 *               is balanced in load and probability).
 * All fp32 outputs on the device. The token sums run over fixed token
 * ranges in a fixed order: deterministic. Logits are assumed finite.
 * T == 0 writes nothing. ws: at least moe_router_workspace_size bytes.
 * MOE_EINVAL on a NULL pointer, MOE_EWORKSPACE if ws is too small. */
moe_status moe_load_balance_stats(const moe_desc* desc, const float* logits,
                                  const int32_t* counts, float* f,
                                  float* p_mean, float* aux, void* ws,
                                  size_t ws_bytes, void* stream);

/* Route-bias step of the auxiliary-loss-free balancing [P3 §6.3, §9],
 * from one routing's counts [E] (e.g. moe_forward's): load[e] =
 * counts[e] / sum(counts), then in fp32, each product and difference
 * rounded once:
 *   rule 0 (the stated rule): bias[e] -= gamma * sign(load[e] - target);
 *   rule 1 (the layer's update_balance_bias variant):
 *          bias[e] -= gamma * sign(load[e] - target) * max(load[e], 1e-6);
 * target <= 0 means 1/E; sign(0) = 0. route_bias [E] fp32 is updated in
 * place (it only moves the selection, see moe_route); load [E] fp32 is
 * written if non-NULL. T == 0 changes nothing. MOE_EINVAL on a NULL
 * counts or route_bias, a rule other than 0 or 1, or a NaN gamma or
 * target. */
moe_status moe_update_route_bias(const moe_desc* desc, const int32_t* counts,
                                 float* route_bias, float gamma, float target,
                                 int32_t rule, float* load, void* stream);

/* Load monitor [P3 §13.9]: from a window of W >= 1 load vectors
 * load_hist [W, E] fp32 (e.g. successive moe_update_route_bias loads,
 * oldest first; the pages average the latest 100), the mean load r (rows
 * summed in order), and out[0] = min r, out[1] = -sum r log(r + 1e-9)
 * (entropy), out[2] = number of experts with r < 0.3 / E (cold experts),
 * all fp32 on the device. MOE_EINVAL on a NULL pointer or W < 1. */
moe_status moe_balance_monitor(const moe_desc* desc, const float* load_hist,
                               int32_t W, float* out, void* stream);

/* Transposing MX quantisation, for the weights of the MXFP8 backward's
 * data-gradient products [P3 §13.6: gradient times transposed weight]:
 * for each of `batch` bf16 [rows, cols] matrices src_b (contiguous),
 *   q_b[c, col_off + r] = E4M3 code of src_b[r, c] in 32-blocks along r,
 * with q_b of row stride ldq (batch stride cols * ldq), and the blocks'
 * E8M0 codes in `scales`, the MX scale layout of the stacked
 * [batch * cols, ldq] operand; same rule as moe_quantize_mxfp8.
 * W2 [E, d, f] -> w2t: (E, d, f, ldq = d, col_off 0); W1, W3 [E, f, d] ->
 * w13t: (E, f, d, ldq = 2 f, col_off 0 and f). rows % 32 == 0,
 * cols % 64 == 0, ldq % 128 == 0, col_off % 128 == 0 and
 * col_off + rows <= ldq, else MOE_EUNSUPPORTED / MOE_EINVAL. */
moe_status moe_quantize_mxfp8_t(const void* src_bf16, int64_t batch,
                                int64_t rows, int64_t cols, uint8_t* q,
                                uint8_t* scales, int64_t ldq, int64_t col_off,
                                void* stream);

/* MX quantisation of a bf16 [rows, cols] matrix along its rows (cols a
 * multiple of 128) [P2 section on the TE mechanisms: MXFP8 grouped GEMM
 * operands; P3 §13.6: fp8 with per-tile rather than per-tensor scales].
 * The pages fix no bit-level rule; this is the OCP MX v1.0 one: X = floor(log2(amax)) - 8
 * per 32-element block (clamped to [-127, 127]); scale code X + 127;
 * element = E4M3 round-to-nearest-even of v / 2^X, saturated to +-448.
 * Writes q [rows, cols] E4M3 bytes and the rows * cols / 32 scale codes
 * in the MX scale layout (device pointers owned by the caller). NULL
 * pointers, rows < 0 or cols <= 0 -> MOE_EINVAL; cols % 128 != 0 ->
 * MOE_EUNSUPPORTED; rows == 0 -> MOE_OK with nothing enqueued. */
moe_status moe_quantize_mxfp8(const void* src_bf16, int64_t rows,
                              int64_t cols, uint8_t* q, uint8_t* scales,
                              void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
