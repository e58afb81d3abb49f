// Drives the host side of the C ABI (include/afd_ffn.h) through every argument check,
// in a build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code,
// without a GPU: a handle is filled in by hand (no device buffers), and every call
// either fails its host checks before enqueuing anything or reaches a HIP call that
// fails for want of a device.  Checks the return codes; exit status 0 and
// "abi driver ok" on success.  Test infrastructure only.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "afd_ffn.h"
#include "afd_internal.h"

static int failures = 0;
#define EXPECT(cond, what)                         \
  do {                                             \
    if (!(cond)) {                                 \
      fprintf(stderr, "FAIL: %s (line %d)\n", what, __LINE__); \
      ++failures;                                  \
    }                                              \
  } while (0)

// Fake device addresses: never dereferenced on the host, only compared and checked for
// alignment and overlap.
static void* addr(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  // ---- configuration and create
  afd_ffn_config cfg = {256, 128, 8, 2, 16, 0, AFD_BF16};
  afd_ffn_t out = nullptr;
  EXPECT(afd_ffn_create(nullptr, addr(0x1000), addr(0x2000), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, &out) == AFD_EINVAL, "NULL config");
  const afd_ffn_config bad[] = {
      {100, 128, 8, 2, 16, 0, AFD_BF16}, {256, 0, 8, 2, 16, 0, AFD_BF16},    {256, 128, 0, 2, 16, 0, AFD_BF16},
      {256, 128, 8, 9, 16, 0, AFD_BF16}, {256, 128, 8, 2, 0, 0, AFD_BF16},     {256, 128, 8, 2, 16, 100, AFD_BF16},
      {256, 128, 8, 2, 16, 0, 7},        {256, 128, 2000, 2, 16, 0, AFD_BF16}, {256, 128, 64, 33, 16, 0, AFD_BF16},
      {256, 128, 8, 8, 1 << 30, 0, AFD_BF16}};
  for (const afd_ffn_config& c : bad)
    EXPECT(afd_ffn_create(&c, addr(0x1000), addr(0x2000), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, &out) == AFD_EINVAL, "bad config refused");
  EXPECT(afd_ffn_create(&cfg, nullptr, addr(0x2000), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        &out) == AFD_EINVAL, "NULL weights");
  EXPECT(afd_ffn_create(&cfg, addr(0x1001), addr(0x2000), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, &out) == AFD_EINVAL, "misaligned weights");
  EXPECT(afd_ffn_create(&cfg, addr(0x1000), addr(0x2000), (const float*)addr(0x3000), nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr, &out) == AFD_EINVAL, "scales on a bf16 layer");
  afd_ffn_config f8 = cfg;
  f8.dtype = AFD_FP8_E4M3;
  EXPECT(afd_ffn_create(&f8, addr(0x1000), addr(0x2000), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, &out) == AFD_EINVAL, "fp8 without scales");
  // valid arguments: without a device, create fails in HIP and returns no handle
  const int rc = afd_ffn_create(&cfg, addr(0x1000), addr(0x2000), nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, &out);
  EXPECT(rc == AFD_EHIP || rc == AFD_OK, "create without a device");
  if (rc == AFD_OK) afd_ffn_destroy(out);
  EXPECT(strlen(afd_ffn_last_error()) > 0, "last_error after a failure");

  // ---- a handle filled in by hand
  afd_ffn* h = new afd_ffn();
  h->cfg = cfg;
  h->device = 0;
  const int T = 16, P = T * 2;
  afd_route r = {(int32_t*)addr(0x10000), (float*)addr(0x20000), (int32_t*)addr(0x30000), (int32_t*)addr(0x40000),
                 (int32_t*)addr(0x50000), (int32_t*)addr(0x60000)};
  const float* logits = (const float*)addr(0x70000);
  EXPECT(afd_ffn_route(h, logits, -1, &r, nullptr) == AFD_EINVAL, "T < 0");
  EXPECT(afd_ffn_route(h, logits, T + 1, &r, nullptr) == AFD_EINVAL, "T > max_tokens");
  EXPECT(afd_ffn_route(h, nullptr, T, &r, nullptr) == AFD_EINVAL, "NULL logits");
  EXPECT(afd_ffn_route(h, logits, T, nullptr, nullptr) == AFD_EINVAL, "NULL route");
  EXPECT(afd_ffn_route(h, (const float*)addr(0x70002), T, &r, nullptr) == AFD_EINVAL, "misaligned logits");
  EXPECT(afd_ffn_route(h, (const float*)addr(0x10000), T, &r, nullptr) == AFD_EINVAL, "logits on the ids");
  EXPECT(afd_ffn_route(h, logits, 0, &r, nullptr) == AFD_OK, "T = 0 is a no-op");
  afd_route ov = r;
  ov.topk_gates = (float*)addr(0x10000 + 4 * P - 4);
  EXPECT(afd_ffn_route(h, logits, T, &ov, nullptr) == AFD_EINVAL, "route buffers overlap");
  afd_route nul = r;
  nul.pair_pos = nullptr;
  EXPECT(afd_ffn_route(h, logits, T, &nul, nullptr) == AFD_EINVAL, "NULL route buffer");
  EXPECT(afd_ffn_route_select_bias(h, logits, nullptr, T, &r, nullptr) == AFD_EINVAL, "NULL bias");
  EXPECT(afd_ffn_route_hidden(h, addr(0x80000), nullptr, nullptr, (float*)addr(0x90000), T, &r, nullptr) ==
             AFD_EINVAL, "NULL router weights");
  EXPECT(afd_ffn_route_hidden(h, addr(0x80000), addr(0xA0000), nullptr, (float*)addr(0x80000), T, &r, nullptr) ==
             AFD_EINVAL, "logits on x");
  // capacity routing
  int32_t* lim = (int32_t*)addr(0xB0000);
  EXPECT(afd_ffn_route_capacity(h, r.topk_ids, r.topk_gates, T, -1, 1, lim, (int32_t*)addr(0xC0000),
                                (float*)addr(0xD0000), (int32_t*)addr(0xE0000), (int32_t*)addr(0xF0000),
                                nullptr) == AFD_EINVAL, "negative base capacity");
  EXPECT(afd_ffn_route_capacity(h, r.topk_ids, r.topk_gates, T, 1, 1, lim, (int32_t*)addr(0xC0000),
                                (float*)addr(0xC0000), (int32_t*)addr(0xE0000), (int32_t*)addr(0xF0000),
                                nullptr) == AFD_EINVAL, "capacity outputs overlap");
  EXPECT(afd_ffn_route_from_capacity(h, nullptr, nullptr, nullptr, nullptr, T, &r, nullptr) == AFD_EINVAL,
         "NULL capacity result");
  // forward and its variants
  void* x = addr(0x100000);
  void* y = addr(0x200000);
  EXPECT(afd_ffn_forward(h, nullptr, T, &r, y, nullptr) == AFD_EINVAL, "NULL x");
  EXPECT(afd_ffn_forward(h, x, T, &r, addr(0x100010), nullptr) == AFD_EINVAL, "x and y overlap");
  EXPECT(afd_ffn_forward(h, addr(0x100004), T, &r, y, nullptr) == AFD_EINVAL, "misaligned x");
  EXPECT(afd_ffn_forward(h, x, T, &r, (void*)r.sorted_pair, nullptr) == AFD_EINVAL, "y on a route buffer");
  EXPECT(afd_ffn_forward(h, x, 0, &r, y, nullptr) == AFD_OK, "forward T = 0");
  EXPECT(afd_ffn_forward_noalloc(h, nullptr, T, &r, y, nullptr) == AFD_EINVAL, "noalloc NULL x");
  EXPECT(afd_ffn_forward_noalloc(h, x, T, &r, addr(0x100010), nullptr) == AFD_EINVAL, "noalloc overlap");
  EXPECT(afd_ffn_forward_fp8_input(h, (const uint8_t*)x, (const float*)addr(0x300000), T, &r, y, nullptr) ==
             AFD_EUNSUPPORTED, "fp8 input on a bf16 layer");
  {  // a layer too large for the no-allocation scratch
    afd_ffn* big = new afd_ffn();
    big->cfg = {4096, 1536, 4, 4, 1500, 0, AFD_BF16};
    big->device = 0;
    EXPECT(afd_ffn_forward_noalloc(big, x, 16, &r, y, nullptr) == AFD_EINVAL, "noalloc beyond the scratch");
    delete big;
  }
  // knobs, profiling, sizes, errors
  EXPECT(afd_ffn_set_gemm_kernel(h, AFD_GEMM_TILED) == AFD_OK, "gemm knob");
  EXPECT(afd_ffn_set_gemm_kernel(h, AFD_GEMM_FUSED) == AFD_OK, "fused knob");
  EXPECT(afd_ffn_set_gemm_kernel(h, 4) == AFD_EINVAL, "unknown gemm kernel");
  EXPECT(afd_ffn_set_profiling(h, 1) == AFD_OK && afd_ffn_set_profiling(h, 0) == AFD_OK, "profiling");
  double ms[AFD_NUM_STAGES];
  int64_t n[AFD_NUM_STAGES];
  EXPECT(afd_ffn_profile_read(h, ms, n, AFD_NUM_STAGES) == AFD_OK, "profile read with no events");
  EXPECT(afd_ffn_profile_read(h, nullptr, n, AFD_NUM_STAGES) == AFD_EINVAL, "profile read NULL");
  EXPECT(afd_ffn_route_bytes(h) == 4 * (4 * (size_t)P + 2 * 8 + 1), "route bytes");
  EXPECT(afd_ffn_route_bytes(nullptr) == 0 && afd_ffn_device_bytes(nullptr) == 0, "NULL sizes");
  EXPECT(afd_ffn_quantize_fp8(x, 4, 100, AFD_BF16, (uint8_t*)y, (float*)addr(0x300000), nullptr) == AFD_EINVAL,
         "quantise ragged columns");
  EXPECT(afd_ffn_quantize_fp8(x, 4, 128, AFD_FP8_E4M3, (uint8_t*)y, (float*)addr(0x300000), nullptr) == AFD_EINVAL,
         "quantise fp8 source");
  EXPECT(afd_ffn_quantize_fp8(x, 0, 128, AFD_BF16, nullptr, nullptr, nullptr) == AFD_OK, "quantise 0 rows");
  for (int c : {AFD_OK, AFD_EINVAL, AFD_EUNSUPPORTED, AFD_ENOMEM, AFD_EHIP, -99})
    EXPECT(afd_ffn_strerror(c) && strlen(afd_ffn_strerror(c)) > 0, "strerror");
  EXPECT(afd_ffn_destroy(nullptr) == AFD_OK, "destroy NULL");
  delete h;  // no device buffers: not afd_ffn_destroy
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi driver ok\n");
  return 0;
}
