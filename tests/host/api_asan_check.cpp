// Host-side memory check of the C ABI's argument validation and workspace
// sizing, built with AddressSanitizer on the host code of csrc/api.cpp.
// Every struct handed to the library is heap-allocated at its exact size,
// so a read past one is caught. Only calls that the validation must reject
// before any device work are made (or the pure size queries), so no GPU is
// needed. Exit status 0 and "OK" on success.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../../include/moe.h"

namespace {

[[noreturn]] void fail(const char* what, int got) {
  std::printf("FAIL %s (status %d)\n", what, got);
  std::exit(1);
}

void expect(moe_status got, moe_status want, const char* what) {
  if (got != want) fail(what, (int)got);
}

moe_desc* make(int T, int d, int f, int E, int K, int fs = 0, int act = MOE_BF16,
               int gemm = MOE_BF16, int gate = MOE_GATE_SOFTMAX, int flags = 0) {
  moe_desc* p = new moe_desc;
  p->T = T; p->d_model = d; p->d_ff = f; p->E = E; p->K = K;
  p->d_ff_shared = fs; p->gate = gate; p->act_dtype = act; p->gemm_dtype = gemm;
  p->flags = flags;
  return p;
}

}  // namespace

int main(int argc, char** argv) {
  const int n_random = argc > 1 ? std::atoi(argv[1]) : 20000;
  void* fake = (void*)(uintptr_t)0x1000;
  size_t bytes = 0;

  // status strings, in and out of range
  for (int s = -3; s < 10; ++s)
    if (!moe_status_str((moe_status)s)) fail("status string", s);

  // size queries: NULL arguments, then random descriptors (valid and not)
  moe_desc* good = make(4096, 1024, 2048, 64, 8, 512);
  expect(moe_workspace_size(nullptr, 0, &bytes), MOE_EINVAL, "size: NULL desc");
  expect(moe_workspace_size(good, 0, nullptr), MOE_EINVAL, "size: NULL out");
  expect(moe_router_workspace_size(nullptr, &bytes), MOE_EINVAL, "router size: NULL");
  std::mt19937 rng(7);
  auto pick = [&](std::initializer_list<int> v) {
    return *(v.begin() + std::uniform_int_distribution<int>(0, (int)v.size() - 1)(rng));
  };
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  long ok = 0;
  for (int i = 0; i < n_random; ++i) {
    moe_desc* d = make(pick({0, 1, 7, 1024, uni(1, 70000), -1}),
                       pick({8, 64, 128, 200, 4096, 7168, 0, 12}),
                       pick({8, 128, 1408, 14336, 0, 30}),
                       pick({1, 4, 6, 8, 60, 256, 1024, 1025, 0}),
                       pick({1, 2, 4, 8, 16, 17, 0}),
                       pick({0, 0, 128, 2816, 13}),
                       pick({MOE_BF16, MOE_F32, 5}),
                       pick({MOE_BF16, MOE_F32, MOE_MXFP8, 7}),
                       pick({MOE_GATE_SOFTMAX, MOE_GATE_SIGMOID, 3}),
                       pick({0, MOE_FLAG_SAVE_ACTS, 0x40000000}));
    for (int bwd = 0; bwd < 2; ++bwd) {
      bytes = 0;
      const moe_status s = moe_workspace_size(d, bwd, &bytes);
      if (s != MOE_OK && s != MOE_EINVAL && s != MOE_EUNSUPPORTED) fail("size status", s);
      if (s == MOE_OK) {
        ++ok;
        if (d->T > 0 && bytes == 0) fail("zero workspace", d->T);
        if (bytes > ((size_t)1 << 42)) fail("absurd workspace", (int)(bytes >> 30));
      }
    }
    const moe_status r = moe_router_workspace_size(d, &bytes);
    if (r != MOE_OK && r != MOE_EINVAL && r != MOE_EUNSUPPORTED) fail("router size status", r);
    delete d;
  }
  if (ok == 0) fail("no valid random descriptor", 0);

  // entry points: rejected before any device work
  moe_desc* bad = make(16, 64, 64, 4, 5);  // K > E
  moe_fwd_args* fa = new moe_fwd_args{};
  moe_bwd_args* ba = new moe_bwd_args{};
  expect(moe_forward(nullptr, fa, fake, 1 << 20, nullptr), MOE_EINVAL, "fwd: NULL desc");
  expect(moe_forward(bad, fa, fake, 1 << 20, nullptr), MOE_EINVAL, "fwd: K > E");
  expect(moe_forward(good, nullptr, fake, 1 << 20, nullptr), MOE_EINVAL, "fwd: NULL args");
  expect(moe_forward(good, fa, fake, 1 << 20, nullptr), MOE_EINVAL, "fwd: NULL buffers");
  expect(moe_forward_noalloc(good, nullptr, nullptr), MOE_EINVAL, "noalloc: NULL args");
  expect(moe_forward_noalloc(bad, fa, nullptr), MOE_EINVAL, "noalloc: K > E");
  expect(moe_backward(good, nullptr, fake, 1 << 20, nullptr), MOE_EINVAL, "bwd: NULL args");
  expect(moe_backward(good, ba, fake, 1 << 20, nullptr), MOE_EINVAL, "bwd: NULL buffers");
  expect(moe_backward(bad, ba, fake, 1 << 20, nullptr), MOE_EINVAL, "bwd: K > E");
  expect(moe_route(nullptr, fake, fake, nullptr, nullptr, (float*)fake, (int32_t*)fake,
                   (float*)fake, nullptr), MOE_EINVAL, "route: NULL desc");
  expect(moe_route(good, fake, fake, nullptr, nullptr, nullptr, (int32_t*)fake,
                   (float*)fake, nullptr), MOE_EINVAL, "route: no logits out");
  expect(moe_permute(good, fake, nullptr, (int32_t*)fake, (int32_t*)fake, (int32_t*)fake,
                     (int32_t*)fake, fake, nullptr, fake, 1 << 20, nullptr),
         MOE_EINVAL, "permute: NULL idx");
  expect(moe_permute(good, fake, (int32_t*)fake, (int32_t*)fake, (int32_t*)fake,
                     (int32_t*)fake, (int32_t*)fake, fake, nullptr, fake, 1, nullptr),
         MOE_EWORKSPACE, "permute: small workspace");
  moe_expert_weights* w = new moe_expert_weights{};
  expect(moe_grouped_gemm_swiglu(good, fake, nullptr, (int32_t*)fake, w, nullptr, nullptr,
                                 fake, fake, nullptr, nullptr, nullptr, fake, 1 << 20, nullptr),
         MOE_EINVAL, "gemm: no weights");
  expect(moe_unpermute_combine(bad, fake, (int32_t*)fake, (float*)fake, nullptr, fake, nullptr),
         MOE_EINVAL, "combine: K > E");
  expect(moe_router_backward(good, fake, fake, nullptr, (int32_t*)fake, (float*)fake,
                             (float*)fake, (int32_t*)fake, 0.0f, (float*)fake, fake, fake,
                             fake, 1 << 20, nullptr),
         MOE_EINVAL, "router bwd: NULL logits");
  expect(moe_load_balance_stats(good, nullptr, (int32_t*)fake, (float*)fake, (float*)fake,
                                (float*)fake, fake, 1 << 20, nullptr),
         MOE_EINVAL, "balance: NULL logits");
  expect(moe_update_route_bias(good, (int32_t*)fake, (float*)fake, 0.001f, 0.0f, 2,
                               (float*)fake, nullptr),
         MOE_EINVAL, "bias: bad rule");
  expect(moe_balance_monitor(good, (float*)fake, 0, (float*)fake, nullptr), MOE_EINVAL,
         "monitor: W = 0");
  expect(moe_quantize_mxfp8(fake, 4, 96, (uint8_t*)fake, (uint8_t*)fake, nullptr),
         MOE_EUNSUPPORTED, "quantize: cols % 128");
  expect(moe_quantize_mxfp8(fake, 4, 128, (uint8_t*)fake, (uint8_t*)fake + 1, nullptr),
         MOE_EINVAL, "quantize: unaligned scales");
  expect(moe_quantize_mxfp8_t(fake, 2, 64, 128, (uint8_t*)fake, (uint8_t*)fake, 192, 64,
                              nullptr),
         MOE_EUNSUPPORTED, "quantize_t: col_off % 128");
  // MXFP8 descriptor with unaligned scale pointers
  moe_desc* mx = make(256, 256, 256, 8, 2, 0, MOE_BF16, MOE_MXFP8);
  moe_expert_weights* mw = new moe_expert_weights{fake, fake, fake, (uint8_t*)fake + 2,
                                                  (uint8_t*)fake, (uint8_t*)fake};
  expect(moe_grouped_gemm_swiglu(mx, fake, (uint8_t*)fake, (int32_t*)fake, mw, nullptr,
                                 nullptr, fake, fake, nullptr, nullptr, nullptr, fake,
                                 1 << 28, nullptr),
         MOE_EINVAL, "mx gemm: unaligned weight scales");
  delete mw; delete mx; delete w; delete fa; delete ba; delete bad; delete good;
  std::printf("OK %d random descriptors, %ld valid sizings\n", n_random, ok);
  return 0;
}
