// Grouped GEMM entry points used by the layer (internal).
#pragma once

#include "common.h"

namespace moe {

// The six products of the layer, each a fixed operand layout/epilogue.
enum GemmOp : int {
  kOpRouter = 0,  // logits[T,E] = x Wr^T                 (fp32 out, 1 group)
  kOpGemm1 = 1,   // h = silu(x_perm W1_e^T) * (x_perm W3_e^T)   (dual B)
  kOpGemm2 = 2,   // y_perm = h W2_e^T
  kOpDgrad2 = 3,  // dh = dy_perm W2_e -> (da, db) via the SwiGLU derivative
  kOpDgrad1 = 4,  // dx_perm = da W1_e + db W3_e          (K-concatenation)
  kOpWgrad = 5,   // dW_e = L_e^T R_e over the expert's rows (ragged K)
  kOpGemm1Mx = 6, // GEMM 1 on MXFP8 operands; h written as MXFP8
  kOpGemm2Mx = 7, // GEMM 2 on MXFP8 operands; y_perm in bf16
  kOpRouterDx = 8,  // dx_router[T,d] = d_logits[T,E] Wr[E,d]   (1 group)
  kOpRouterDw = 9,  // part_g[E,d] = d_logits_g^T x_g over token range g (fp32)
  kOpGemm1MxAct = 10,  // GEMM 1 on MXFP8 operands; bf16 h (optional), a, b
  kOpDgrad2Mx = 11,    // dh = dy_perm W2_e on MXFP8 operands -> (da, db) bf16
};

// Row-tile heights for which the permute step publishes tile prefixes.
constexpr int kNumTileBM = 4;
constexpr int kTileBM[kNumTileBM] = {32, 64, 128, 256};
__host__ __device__ constexpr int tile_bm_slot(int bm) {
  return bm == 32 ? 0 : bm == 64 ? 1 : bm == 128 ? 2 : 3;
}

// SIMT kernels (fp32 or bf16 operands, any shape; K % 1 == 0).
hipError_t gemm_simt(GemmOp op, int dtype, const GemmParams& p,
                     hipStream_t s);
constexpr int kSimtBM = 64;

// MFMA kernels (bf16 operands). Returns hipErrorNotSupported when the
// shape is outside what the MFMA tiles handle; the caller then uses SIMT.
// `tile_off_by_bm` holds the device tile prefixes for every kTileBM.
hipError_t gemm_mfma(GemmOp op, GemmParams p,
                     const int32_t* const* tile_off_by_bm, hipStream_t s);
bool mfma_supported(GemmOp op, const GemmParams& p);
// Whether the direct-to-LDS kernels are in use (not forced off).
bool gemm_direct_ok();
// Whether GEMM 1 can gather its A rows (direct-to-LDS kernel, bf16 or
// MXFP8) for contraction length K.
bool gemm1_gather_supported(int K);

}  // namespace moe
