// Host-side checks of the C ABI (include/moe.h) for a build whose host code is
// instrumented with AddressSanitizer and UndefinedBehaviorSanitizer. Every call
// here returns before anything is enqueued: queries, workspace sizing, and
// argument validation with null, misaligned or out-of-range arguments. Device
// pointers are placeholders that are never dereferenced, so the program refuses
// to run where a GPU is visible (a validation bug must not become a launch).
// Exit status 0 when every status code is the expected one.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define EXPECT(call, want)                                                                   \
  do {                                                                                       \
    const long long got_ = static_cast<long long>(call);                                     \
    if (got_ != static_cast<long long>(want)) {                                              \
      fprintf(stderr, "line %d: %s returned %lld, expected %lld\n", __LINE__, #call, got_,   \
              static_cast<long long>(want));                                                 \
      ++failures;                                                                            \
    }                                                                                        \
  } while (0)

static moe_dims_t dims(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t dtype = MOE_DTYPE_BF16) {
  moe_dims_t m;
  m.T = T, m.d = d, m.f = f, m.E = E, m.k = k, m.dtype = dtype;
  return m;
}

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    printf("a GPU is visible: the host-only checks do not run here\n");
    return 0;
  }
  void* const A = reinterpret_cast<void*>(uintptr_t(0x10000));   // 16-byte aligned placeholder
  void* const M2 = reinterpret_cast<void*>(uintptr_t(0x10002));  // misaligned placeholder
  const size_t BIG = size_t(1) << 40;

  // status strings: every code, and codes outside the enum
  for (int st = -3; st < 9; ++st) {
    const char* s = moe_status_string(st);
    if (!s || !s[0]) ++failures;
  }
  EXPECT(moe_version() >= 100, 1);

  // workspace sizing: valid shapes grow with T; invalid dims give 0 (no overflow on the way)
  const moe_dims_t prefill = dims(8192, 6144, 16384, 8, 2), decode = dims(256, 6144, 16384, 8, 2);
  EXPECT(moe_workspace_bytes(&prefill) > moe_workspace_bytes(&decode), 1);
  EXPECT(moe_workspace_bytes(&decode) > 0, 1);
  const moe_dims_t bad[] = {dims(64, 128, 256, 8, 0), dims(64, 128, 256, 8, 9), dims(64, 128, 256, 1025, 2),
                            dims(64, 0, 256, 8, 2), dims(64, 128, 0, 8, 2), dims(-1, 128, 256, 8, 2),
                            dims(64, 128, 256, 8, 2, 7), dims(int64_t(1) << 30, 128, 256, 8, 4),
                            dims(int64_t(1) << 40, 128, 256, 8, 2), dims(64, int64_t(1) << 31, 256, 8, 2),
                            dims(int64_t(1) << 62, 1, 1, 1024, 1024)};
  for (const moe_dims_t& b : bad) {
    EXPECT(moe_workspace_bytes(&b), 0);
    EXPECT(moe_workspace_bytes_shared(&b, 1), 0);
    EXPECT(moe_backward_workspace_bytes(&b), 0);
    EXPECT(moe_ffn_block_rows(&b), 0);
    EXPECT(moe_gate_on_matrix_cores(&b), -1);
  }
  EXPECT(moe_workspace_bytes(nullptr), 0);
  EXPECT(moe_ffn_block_rows(&decode), 128);
  EXPECT(moe_ffn_block_rows(&prefill), 256);
  EXPECT(moe_gate_on_matrix_cores(&prefill), 0);
  const moe_dims_t deepseek = dims(4096, 7168, 2048, 256, 8);
  EXPECT(moe_gate_on_matrix_cores(&deepseek), 1);
  const moe_dims_t widest = dims(2000000, 64, 64, 1024, 1024);   // T*k just under 2^31
  EXPECT(moe_workspace_bytes(&widest) > 0, 1);
  const moe_dims_t big_e = dims(4096, 7168, 2048, 1024, 8);
  EXPECT(moe_workspace_bytes_shared(&big_e, 1), 0);             // E + n_shared > 1024
  EXPECT(moe_workspace_bytes_shared(&decode, 2) > moe_workspace_bytes_shared(&decode, 1), 1);

  // tile plan layout: inside the workspace, for plain and shared-expert layers
  size_t mo = 0, co = 0;
  int64_t mx = 0;
  EXPECT(moe_layer_plan_layout(&prefill, 0, &mo, &co, &mx), MOE_OK);
  EXPECT(mo + 16 * size_t(mx) <= co && co + 4 <= moe_workspace_bytes(&prefill), 1);
  EXPECT(moe_layer_plan_layout(&decode, 3, &mo, &co, &mx), MOE_OK);
  EXPECT(co + 4 <= moe_workspace_bytes_shared(&decode, 3), 1);
  EXPECT(moe_layer_plan_layout(&decode, -1, &mo, &co, &mx), MOE_ERR_INVALID);
  EXPECT(moe_layer_plan_layout(&decode, 0, nullptr, &co, &mx), MOE_ERR_INVALID);
  EXPECT(moe_layer_plan_layout(&bad[0], 0, &mo, &co, &mx), MOE_ERR_INVALID);

  // route
  const moe_dims_t small = dims(64, 128, 256, 8, 2);
  EXPECT(moe_route(&small, nullptr, A, nullptr, nullptr, (int32_t*)A, (float*)A, A, BIG, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_route(&small, M2, A, nullptr, nullptr, (int32_t*)A, (float*)A, A, BIG, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_route(&small, A, A, nullptr, nullptr, (int32_t*)A, (float*)A, A, 16, nullptr), MOE_ERR_WORKSPACE);
  const moe_dims_t d100 = dims(64, 100, 256, 8, 2);
  EXPECT(moe_route(&d100, A, A, nullptr, nullptr, (int32_t*)A, (float*)A, A, BIG, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route(&bad[0], A, A, nullptr, nullptr, (int32_t*)A, (float*)A, A, BIG, nullptr), MOE_ERR_INVALID);

  // permute, grouped FFN, combine
  EXPECT(moe_permute(&small, (int32_t*)A, nullptr, (int32_t*)A, (int32_t*)A, (int32_t*)A, A, BIG, nullptr),
         MOE_ERR_INVALID);
  EXPECT(moe_permute(&small, (int32_t*)A, (int32_t*)A, (int32_t*)A, (int32_t*)A, (int32_t*)A, A, 4, nullptr),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_grouped_ffn(&small, A, (int32_t*)A, (int32_t*)A, (int32_t*)A, A, M2, A, A, A, BIG, nullptr),
         MOE_ERR_INVALID);
  const moe_dims_t f96 = dims(64, 128, 96, 8, 2);
  EXPECT(moe_grouped_ffn(&f96, A, (int32_t*)A, (int32_t*)A, (int32_t*)A, A, A, A, A, A, BIG, nullptr),
         MOE_ERR_UNSUPPORTED);
  const moe_dims_t huge_x = dims(int64_t(1) << 26, 128, 256, 8, 2);  // x over 4 GiB
  EXPECT(moe_grouped_ffn(&huge_x, A, (int32_t*)A, (int32_t*)A, (int32_t*)A, A, A, A, A, A, BIG, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_combine(&small, A, (int32_t*)A, (float*)A, nullptr, nullptr), MOE_ERR_INVALID);
  const moe_dims_t d12 = dims(64, 12, 256, 8, 2);
  EXPECT(moe_combine(&d12, A, (int32_t*)A, (float*)A, A, nullptr), MOE_ERR_UNSUPPORTED);

  // the layer entry points
  auto layer = [&](const moe_dims_t* m, void* w2, void* out, void* ws, size_t wsb) {
    return moe_layer_forward(m, A, A, nullptr, A, A, w2, out, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                             nullptr, ws, wsb, nullptr);
  };
  EXPECT(layer(&small, nullptr, A, A, BIG), MOE_ERR_INVALID);
  EXPECT(layer(&small, A, (char*)A + 8, A, BIG), MOE_ERR_INVALID);
  const moe_dims_t d96 = dims(64, 96, 256, 8, 2);
  EXPECT(layer(&d96, A, A, A, BIG), MOE_ERR_UNSUPPORTED);
  EXPECT(layer(&small, A, A, A, 1024), MOE_ERR_WORKSPACE);
  EXPECT(layer(&small, A, A, nullptr, 0), MOE_ERR_WORKSPACE);
  EXPECT(layer(&small, A, A, (char*)A + 64, BIG), MOE_ERR_INVALID);
  const moe_dims_t empty = dims(0, 128, 256, 8, 2);
  EXPECT(layer(&empty, A, A, A, BIG), MOE_OK);
  const moe_dims_t f32 = dims(64, 128, 256, 8, 2, MOE_DTYPE_F32);
  EXPECT(moe_layer_forward_fused(&f32, A, A, nullptr, A, A, A, A, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                 nullptr, A, BIG, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_layer_forward_packed(&f32, A, A, nullptr, A, A, A, A, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, A, BIG, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_layer_forward_fused_packed(&f32, A, A, nullptr, A, A, A, A, nullptr, nullptr, nullptr, nullptr,
                                        nullptr, nullptr, nullptr, A, BIG, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_layer_forward_fused_packed(&small, A, A, nullptr, A, A, A, A, nullptr, nullptr, nullptr, nullptr,
                                        nullptr, nullptr, nullptr, A, 1024, nullptr),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_layer_forward_shared(&small, 0, A, A, nullptr, A, A, A, A, A, A, A, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, A, BIG, nullptr),
         MOE_ERR_INVALID);
  EXPECT(moe_layer_forward_shared(&small, 1, A, A, nullptr, A, A, A, nullptr, A, A, A, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, nullptr, A, BIG, nullptr),
         MOE_ERR_INVALID);
  EXPECT(moe_layer_forward_noalloc(&prefill, A, A, nullptr, A, A, A, A, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr),
         MOE_ERR_SCRATCH);
  EXPECT(moe_layer_forward_noalloc(&bad[1], A, A, nullptr, A, A, A, A, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, nullptr),
         MOE_ERR_INVALID);
  int32_t flags = 7;
  EXPECT(moe_fused_status(&small, A, BIG, nullptr, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_fused_status(&small, A, 16, &flags, nullptr), MOE_ERR_WORKSPACE);
  EXPECT(moe_fused_status(&empty, nullptr, 0, &flags, nullptr), MOE_OK);
  EXPECT(flags, 0);

  // weight re-layout
  EXPECT(moe_pack_weights(&f32, A, A, A, A, A, A, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_pack_weights(&small, A, A, A, nullptr, A, A, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_pack_weights_transposed(&small, A, A, M2, A, A, A, nullptr), MOE_ERR_INVALID);
  const moe_dims_t d100b = dims(64, 100, 256, 8, 2);
  EXPECT(moe_pack_weights_transposed(&d100b, A, A, A, A, A, A, nullptr), MOE_ERR_UNSUPPORTED);

  // backward
  const moe_dims_t bw = dims(64, 256, 512, 8, 2);
  auto backward = [&](const moe_dims_t* m, float* dw1, float* dlogits, size_t wsb) {
    return moe_layer_backward(m, A, A, A, A, A, (int32_t*)A, (float*)A, (int32_t*)A, (int32_t*)A, (int32_t*)A,
                              (int32_t*)A, A, A, (float*)A, (float*)A, dw1, (float*)A, (float*)A, dlogits, nullptr, A,
                              wsb, nullptr);
  };
  const moe_dims_t bw_f32 = dims(64, 256, 512, 8, 2, MOE_DTYPE_F32), bw_d = dims(64, 192, 512, 8, 2);
  EXPECT(backward(&bw_f32, (float*)A, nullptr, BIG), MOE_ERR_UNSUPPORTED);
  EXPECT(backward(&bw_d, (float*)A, nullptr, BIG), MOE_ERR_UNSUPPORTED);
  EXPECT(backward(&bw, nullptr, nullptr, BIG), MOE_ERR_INVALID);
  EXPECT(backward(&bw, (float*)A, (float*)M2, BIG), MOE_ERR_INVALID);
  EXPECT(backward(&bw, (float*)A, nullptr, 16), MOE_ERR_WORKSPACE);

  // training pair and the backward's options
  auto train = [&](const moe_dims_t* m, void* gu, size_t wsb) {
    return moe_layer_forward_train(m, A, A, nullptr, A, A, A, A, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, gu, A, wsb, nullptr);
  };
  EXPECT(train(&bw, nullptr, BIG), MOE_ERR_INVALID);
  EXPECT(train(&bw, M2, BIG), MOE_ERR_INVALID);
  EXPECT(train(&bw_f32, A, BIG), MOE_ERR_UNSUPPORTED);
  EXPECT(train(&bw_d, A, BIG), MOE_ERR_UNSUPPORTED);
  EXPECT(train(&bw, A, 16), MOE_ERR_WORKSPACE);
  auto saved = [&](const moe_dims_t* m, const void* gu, size_t wsb) {
    return moe_layer_backward_saved(m, A, A, A, A, A, (int32_t*)A, (float*)A, (int32_t*)A, (int32_t*)A, (int32_t*)A,
                                    (int32_t*)A, A, gu, A, (float*)A, (float*)A, (float*)A, (float*)A, (float*)A,
                                    nullptr, nullptr, A, wsb, nullptr);
  };
  EXPECT(saved(&bw, nullptr, BIG), MOE_ERR_INVALID);
  EXPECT(saved(&bw, M2, BIG), MOE_ERR_INVALID);
  EXPECT(saved(&bw_f32, A, BIG), MOE_ERR_UNSUPPORTED);
  EXPECT(saved(&bw, A, 16), MOE_ERR_WORKSPACE);
  auto ex = [&](const moe_dims_t* m, const void* gu, int wdt, size_t wsb) {
    return moe_layer_backward_ex(m, A, A, A, A, A, (int32_t*)A, (float*)A, (int32_t*)A, (int32_t*)A, (int32_t*)A,
                                 (int32_t*)A, A, gu, wdt, A, (float*)A, (float*)A, A, A, A, nullptr, nullptr, A, wsb,
                                 nullptr);
  };
  EXPECT(ex(&bw, nullptr, 7, BIG), MOE_ERR_INVALID);
  EXPECT(ex(&bw, M2, MOE_DTYPE_BF16, BIG), MOE_ERR_INVALID);
  EXPECT(ex(&bw_d, nullptr, MOE_DTYPE_BF16, BIG), MOE_ERR_UNSUPPORTED);
  EXPECT(ex(&bw, A, MOE_DTYPE_F32, 16), MOE_ERR_WORKSPACE);

  // stage timing and probes
  EXPECT(moe_timing_enable(0, 0), MOE_ERR_INVALID);
  EXPECT(moe_timing_read(99, nullptr, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_timing_disable(), MOE_OK);
  EXPECT(moe_probe_hbm_read(nullptr, 1 << 20, (int32_t*)A, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_probe_hbm_read(A, 100, (int32_t*)A, nullptr), MOE_ERR_INVALID);
  EXPECT(moe_probe_mfma(0, (float*)A, nullptr), MOE_ERR_INVALID);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("all host-side ABI checks passed\n");
  return 0;
}
