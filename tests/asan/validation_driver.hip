// Drives every C-ABI entry point through its argument checks on the host
// (no GPU, no kernel launch: the launchers are counting stubs), built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code.  Pointers
// handed in are never dereferenced by a rejected call; the ones that pass
// validation point at host memory of the documented size.  Exits non-zero on
// the first status that differs from the documented one.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <climits>
#include <vector>

#include "moeq.h"

extern int g_launches;

static int failures = 0;
#define EXPECT(call, want)                                                                 \
  do {                                                                                     \
    const int got_ = (call);                                                               \
    if (got_ != (want)) {                                                                  \
      fprintf(stderr, "%s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #call, got_, (want)); \
      ++failures;                                                                          \
    }                                                                                      \
  } while (0)

// a host buffer of n bytes, 256-byte aligned
static void* buf(size_t n) {
  void* p = aligned_alloc(256, (n + 255) / 256 * 256 + 256);
  memset(p, 0, (n + 255) / 256 * 256 + 256);
  return p;
}

int main() {
  const int E = 4, H = 256, I = 128, K = 2, T = 8;
  std::vector<void*> owned;
  auto B = [&](size_t n) { void* p = buf(n); owned.push_back(p); return p; };

  // status strings and the codebook
  for (int s = 1; s >= -9; --s) {
    const char* str = moeq_status_string(s);
    if (!str || !*str) { fprintf(stderr, "empty status string %d\n", s); ++failures; }
  }
  EXPECT(moeq_nf4_codebook(nullptr), MOEQ_EINVAL);
  float cb[16];
  EXPECT(moeq_nf4_codebook(cb), MOEQ_OK);
  EXPECT(moeq_abi_version(), MOEQ_ABI_VERSION);

  moeq_qweight gu = {MOEQ_FMT_NF4, E, 2 * I, H, 64, B((size_t)E * 2 * I * H / 2), (float*)B((size_t)E * 2 * I * H / 64 * 4), nullptr};
  moeq_qweight dn = {MOEQ_FMT_NF4, E, H, I, 64, B((size_t)E * H * I / 2), (float*)B((size_t)E * H * I / 64 * 4), nullptr};
  uint16_t* w = (uint16_t*)B((size_t)E * 2 * I * H * 2);
  uint16_t* x = (uint16_t*)B((size_t)T * H * 2);
  int32_t* idx = (int32_t*)B((size_t)T * K * 4);
  float* wts = (float*)B((size_t)T * K * 4);
  uint16_t* out = (uint16_t*)B((size_t)T * H * 2);

  // quantize: descriptor checks
  EXPECT(moeq_quantize_nf4(w, nullptr, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_quantize_nf4(nullptr, &gu, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_quantize_nf4((const uint16_t*)((char*)w + 2), &gu, nullptr), MOEQ_EALIGN);
  moeq_qweight bad = gu;
  bad.blocksize = 32;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EBLOCK);
  bad = gu; bad.cols = 100;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EBLOCK);
  bad = gu; bad.format = 9;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EFORMAT);
  bad = gu; bad.format = MOEQ_FMT_INT8_ROWWISE; bad.blocksize = bad.cols;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EFORMAT);
  bad = gu; bad.num_experts = 0;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EINVAL);
  bad = gu; bad.rows = -3;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EINVAL);
  bad = gu; bad.qdata = nullptr;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EINVAL);
  bad = gu; bad.scales = (float*)((char*)gu.scales + 4);
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EALIGN);
  bad = gu; bad.scale_codes = (uint8_t*)B(64);
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EINVAL);          // codes on a plain NF4 tensor
  bad = gu; bad.format = MOEQ_FMT_NF4_DQ;
  EXPECT(moeq_quantize_nf4(w, &bad, nullptr), MOEQ_EINVAL);          // NF4_DQ without codes
  EXPECT(moeq_stream_reference(w, &bad, nullptr), MOEQ_EFORMAT);
  moeq_qweight i8 = {MOEQ_FMT_INT8_ROWWISE, E, H, I, I, B((size_t)E * H * I), (float*)B((size_t)E * H * 4), nullptr};
  EXPECT(moeq_quantize_int8_rowwise(w, &gu, nullptr), MOEQ_EFORMAT);
  bad = i8; bad.blocksize = 64;
  EXPECT(moeq_quantize_int8_rowwise(w, &bad, nullptr), MOEQ_EBLOCK);
  bad = i8; bad.cols = 12; bad.blocksize = 12;
  EXPECT(moeq_quantize_int8_rowwise(w, &bad, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_dequantize(&gu, nullptr, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_dequantize(&gu, (uint16_t*)((char*)w + 8), nullptr), MOEQ_EALIGN);
  EXPECT(moeq_compress_absmax(&gu, &gu, nullptr), MOEQ_EFORMAT);
  EXPECT(moeq_qweight_copy_async(&gu, &dn, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_qweight_copy_async(&gu, &i8, nullptr), MOEQ_EFORMAT);
  if (g_launches != 0) { fprintf(stderr, "a rejected call launched work\n"); ++failures; }

  // workspace queries: extreme sizes are refused with 0, never overflow
  EXPECT((int)(moeq_experts_forward_workspace_bytes(T, K, &gu, &dn) > 0), 1);
  EXPECT((int)moeq_experts_forward_workspace_bytes(INT_MAX, INT_MAX, &gu, &dn), 0);
  EXPECT((int)moeq_experts_forward_workspace_bytes(-1, K, &gu, &dn), 0);
  EXPECT((int)moeq_experts_forward_workspace_bytes(T, 0, &gu, &dn), 0);
  EXPECT((int)moeq_experts_forward_workspace_bytes(T, K, &gu, &gu), 0);
  EXPECT((int)moeq_experts_forward_workspace_bytes(T, K, nullptr, &dn), 0);
  EXPECT((int)moeq_experts_backward_workspace_bytes(INT_MAX, 1, &gu, &dn), 0);
  EXPECT((int)moeq_route_workspace_bytes(INT_MAX, INT_MAX, E), 0);
  EXPECT((int)moeq_route_workspace_bytes(T, K, MOEQ_MAX_EXPERTS + 1), 0);
  EXPECT((int)moeq_router_route_workspace_bytes(T, H, E, 65), 0);
  EXPECT((int)moeq_router_route_workspace_bytes(INT_MAX, H, E, K), 0);
  EXPECT((int)(moeq_router_route_workspace_bytes(T, H, E, K) > 0), 1);

  // forward / backward argument checks
  const size_t need = moeq_experts_forward_workspace_bytes(T, K, &gu, &dn);
  void* ws = B(need);
  EXPECT(moeq_experts_forward(x, idx, wts, T, K, &gu, &dn, out, ws, need - 1, nullptr), MOEQ_EWORKSPACE);
  EXPECT(moeq_experts_forward(x, idx, wts, T, K, &gu, &dn, out, nullptr, need, nullptr), MOEQ_EWORKSPACE);
  EXPECT(moeq_experts_forward(nullptr, idx, wts, T, K, &gu, &dn, out, ws, need, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_experts_forward(x, idx, wts, T, K, &gu, &i8, out, ws, need, nullptr), MOEQ_EFORMAT);
  EXPECT(moeq_experts_forward(x, idx, wts, T, K, &dn, &gu, out, ws, need, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_experts_forward(x, idx, wts, T, 0, &gu, &dn, out, ws, need, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_experts_forward(x, idx, wts, (1 << 24) + 1, 1, &gu, &dn, out, ws, need, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_experts_forward((const uint16_t*)((char*)x + 2), idx, wts, T, K, &gu, &dn, out, ws, need, nullptr),
         MOEQ_EALIGN);
  EXPECT(moeq_experts_forward(x, idx, wts, 0, K, &gu, &dn, nullptr, nullptr, 0, nullptr), MOEQ_OK);  // T = 0
  EXPECT(moeq_experts_forward_routed(x, idx, wts, T, K, &gu, &dn, nullptr, idx, idx, out, ws, need, nullptr),
         MOEQ_EINVAL);
  const size_t bneed = moeq_experts_backward_workspace_bytes(T, K, &gu, &dn);
  void* bws = B(bneed);
  EXPECT(moeq_experts_backward(x, idx, wts, T, K, &gu, &dn, x, out, wts, bws, bneed - 1, nullptr), MOEQ_EWORKSPACE);
  EXPECT(moeq_experts_backward(x, idx, wts, T, K, &gu, &dn, nullptr, out, wts, bws, bneed, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_router_topk(x, x, T, H, E, E + 1, 0, idx, wts, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_router_topk(x, x, T, 100, E, K, 0, idx, wts, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_router_topk(x, x, T, H, MOEQ_MAX_EXPERTS + 1, K, 0, idx, wts, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_router_topk(nullptr, x, T, H, E, K, 0, idx, wts, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_router_route(x, x, T, H, E, 65, 0, idx, wts, idx, idx, idx, idx, ws, need, nullptr), MOEQ_ESHAPE);
  EXPECT(moeq_router_route(x, x, T, H, E, K, 0, idx, wts, nullptr, idx, idx, idx, ws, need, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_route_buckets(idx, T, K, E, nullptr, idx, idx, idx, ws, need, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_route_buckets(idx, T, K, 0, idx, idx, idx, idx, ws, need, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_experts_forward_noalloc(x, idx, wts, T, 0, &gu, &dn, out, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_experts_forward_noalloc(x, idx, wts, 0, K, &gu, &dn, nullptr, nullptr), MOEQ_OK);
  EXPECT(moeq_experts_forward_noalloc(nullptr, idx, wts, T, K, &gu, &dn, out, nullptr), MOEQ_EINVAL);
  EXPECT(moeq_experts_forward_noalloc(x, idx, wts, 1 << 20, K, &gu, &dn, out, nullptr), MOEQ_EWORKSPACE);
  if (g_launches != 0) { fprintf(stderr, "a rejected call launched work (%d)\n", g_launches); ++failures; }

  // calls that pass validation reach exactly their launchers (stubs here)
  EXPECT(moeq_quantize_nf4(w, &gu, nullptr), MOEQ_OK);
  EXPECT(moeq_experts_forward(x, idx, wts, T, K, &gu, &dn, out, ws, need, nullptr), MOEQ_OK);
  if (g_launches != 2) { fprintf(stderr, "expected 2 launcher calls, got %d\n", g_launches); ++failures; }

  for (void* p : owned) free(p);
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("validation driver: all checks passed\n");
  return failures ? 1 : 0;
}
