// The C ABI's argument validation over its rejection cases, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code by
// tests/test_sanitize_cpu.py.  Every call below fails validation before the
// library makes any HIP call (the pointers are fake addresses, never
// dereferenced); the workspace queries and status strings run too.  Exit
// status 0 when every call returned the expected code.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hocf.h"

static int fails = 0;
#define EXPECT(c)                                                                   \
  do {                                                                              \
    if (!(c)) {                                                                     \
      std::fprintf(stderr, "FAIL line %d: %s (%s)\n", __LINE__, #c, hocf_last_error()); \
      ++fails;                                                                      \
    }                                                                               \
  } while (0)

// each named buffer its own 1 TiB region of fake device addresses
static void* fake(int i) { return reinterpret_cast<void*>((uintptr_t)((1ull << 44) + ((uint64_t)i << 40))); }
static uint32_t* fake32(int i) { return static_cast<uint32_t*>(fake(i)); }

int main() {
  const hocf_status INV = HOCF_ERR_INVALID_ARG, UNS = HOCF_ERR_UNSUPPORTED;
  EXPECT(hocf_abi_version() == HOCF_ABI_VERSION);
  for (int s = -1; s <= 10; ++s) EXPECT(hocf_status_string(static_cast<hocf_status>(s)) != nullptr);
  EXPECT(hocf_last_error() != nullptr);
  EXPECT(hocf_gemm_rs_workspace_bytes(8, 8192, 4096, 256, 256) > 0);
  EXPECT(hocf_gemm_rs_workspace_bytes(0, 8192, 4096, 256, 256) == 0);
  EXPECT(hocf_gemm_ar_workspace_bytes(8, 8192, 4096, 256, 256) > 0);
  EXPECT(hocf_gemv_ar_workspace_bytes(8, 8192, 256) > 0);
  EXPECT(hocf_ag_gemm_workspace_bytes(8) > 0);
  EXPECT(hocf_embbag_a2a_workspace_bytes() > 0);
  EXPECT(hocf_gemm_a2a_workspace_bytes(8) > 0);
  EXPECT(hocf_a2a_gemm_workspace_bytes(8, 4, 4096, 2, 12288, 256) > 0);
  EXPECT(hocf_a2a_gemm_workspace_bytes(-1, 4, 4096, 2, 12288, 256) == 0);

  hocf_window win[HOCF_MAX_P];
  for (int r = 0; r < HOCF_MAX_P; ++r) { win[r].data = fake(20 + r); win[r].flags = fake32(40 + r); }
  hocf_sync s{};
  s.epoch = 1;
  s.workspace = fake(60);
  s.workspace_bytes = 1 << 24;
  s.status = fake32(61);
  hocf_sync zero_epoch = s;
  zero_epoch.epoch = 0;
  hocf_sync small_ws = s;
  small_ws.workspace_bytes = 8;
  const hocf_dtype F = HOCF_F32, H = HOCF_BF16;

  // GEMM + ReduceScatter / AllReduce / unfused / no-alloc / decomposed
  EXPECT(hocf_gemm_rs(0, 256, 256, 256, F, F, F, fake(1), fake(2), win, fake(3), 64, 64, &s, nullptr) == INV);
  EXPECT(hocf_gemm_rs(4, 256, 256, 256, F, F, F, fake(1), fake(2), win, fake(3), 64, 64, nullptr, nullptr) == INV);
  EXPECT(hocf_gemm_rs(4, 256, 256, 256, F, F, F, fake(1), fake(2), win, fake(3), 64, 64, &zero_epoch, nullptr) == INV);
  EXPECT(hocf_gemm_rs(4, 256, 256, 256, F, F, F, fake(1), fake(2), win, fake(3), 64, 64, &small_ws, nullptr) == INV);
  EXPECT(hocf_gemm_rs(4, 254, 256, 256, F, F, F, fake(1), fake(2), win, fake(3), 64, 64, &s, nullptr) == INV);
  EXPECT(hocf_gemm_rs(4, 256, 256, 256, F, F, F, fake(1), fake(2), nullptr, fake(3), 64, 64, &s, nullptr) == INV);
  EXPECT(hocf_gemm_rs(4, 256, 256, 256, F, F, F, fake(1), fake(2), win, fake(1), 64, 64, &s, nullptr) == INV);
  EXPECT(hocf_gemm_rs(4, 256, 256, 256, H, F, H, fake(1), fake(2), win, fake(3), 96, 96, &s, nullptr) == UNS);
  EXPECT(hocf_gemm_rs_unfused(4, 256, 256, 256, F, F, F, nullptr, fake(2), win, fake(3), 64, 64, &s, nullptr) == INV);
  EXPECT(hocf_gemm_rs_noalloc(4, 256, 256, 256, F, F, F, fake(1), fake(2), win, fake(3), 64, 64, &s, nullptr) == INV);
  EXPECT(hocf_gemm_rs_decomposed(4, 256, 256, 256, F, F, F, fake(1), fake(2), win, fake(3), 64, 64, 0, 0, &s,
                                 nullptr, nullptr) == INV);
  void* outs[HOCF_MAX_P];
  for (int q = 0; q < HOCF_MAX_P; ++q) outs[q] = fake(70 + q);
  outs[1] = outs[0];  // two outputs alias
  EXPECT(hocf_gemm_ar(4, 256, 256, 256, F, F, F, fake(1), fake(2), win, outs, 64, 64, &s, nullptr) == INV);
  const hocf_dtype BAD = static_cast<hocf_dtype>(5);  // no such dtype (any int may arrive from C)
  EXPECT(hocf_gemm_rs(4, 256, 256, 256, BAD, F, F, fake(1), fake(2), win, fake(3), 64, 64, &s, nullptr) == INV);
  EXPECT(hocf_gemv_ar(8, 4, 8192, 1024, H, F, static_cast<hocf_dtype>(-1), fake(1), fake(2), fake(3), fake32(4), win,
                      256, &s, nullptr) == INV);
  EXPECT(hocf_ag_gemm(8, 1024, 1792, 4096, BAD, H, fake(1), fake32(2), fake(3), fake(4), 256, 256, &s, nullptr) ==
         INV);
  // GEMV + AllReduce
  EXPECT(hocf_gemv_ar(8, 4, 8192, 1024, H, F, H, fake(1), fake(2), fake(3), fake32(4), win, 100, &s, nullptr) != HOCF_OK);
  EXPECT(hocf_gemv_ar(8, 4, 8192, 1024, H, F, H, fake(1), fake(2), fake(1), fake32(4), win, 256, &s, nullptr) == INV);
  EXPECT(hocf_gemv_ar_unfused(0, 4, 8192, 1024, H, F, H, fake(1), fake(2), fake(3), fake32(4), win, 256, &s,
                              nullptr) == INV);
  // AllGather + GEMM
  EXPECT(hocf_ag_gemm(8, 1024, 1792, 4096, F, H, fake(1), fake32(2), fake(3), fake(4), 256, 256, &s, nullptr) == UNS);
  EXPECT(hocf_ag_gemm(8, 1024, 1792, 4096, H, H, fake(1), fake32(2), fake(3),
                      static_cast<char*>(fake(1)) + 4096, 256, 256, &s, nullptr) == INV);
  EXPECT(hocf_ag_gemm(8, 1024, 1 << 22, 4096, H, F, fake(1), fake32(2), fake(3), fake(4), 256, 256, &s, nullptr) ==
         UNS);
  // embedding bag + All-to-All
  EXPECT(hocf_embbag_a2a(64, 1000000, 516, 16384, 20, 8, static_cast<float*>(fake(1)),
                         static_cast<int32_t*>(fake(2)), nullptr, win, 64, &s, nullptr) == UNS);
  EXPECT(hocf_embbag_a2a(64, 1000000, 128, 16384, 20, 8, static_cast<float*>(fake(1)),
                         static_cast<int32_t*>(fake(2)), nullptr, win, 0, &s, nullptr) == INV);
  // MoE combine and dispatch
  EXPECT(hocf_gemm_a2a(8, 4, 8192, 4096, 1792, H, H, nullptr, fake(2), nullptr, static_cast<int32_t*>(fake(3)),
                       static_cast<int32_t*>(fake(4)), nullptr, win, 12288, 256, 256, &s, nullptr) == INV);
  EXPECT(hocf_a2a_gemm(8, 4, 0, 4096, 2, 1792, 4096, H, H, static_cast<char*>(fake(1)) + 8,
                       static_cast<int32_t*>(fake(2)), fake(3), 12288, fake(4), fake(5),
                       static_cast<int64_t*>(fake(6)), static_cast<int32_t*>(fake(7)),
                       static_cast<int32_t*>(fake(8)), static_cast<int64_t*>(fake(9)), 256, 256, &s,
                       nullptr) == INV);
  EXPECT(hocf_a2a_gemm_unfused(0, 4, 0, 4096, 2, 1792, 4096, H, H, fake(1), static_cast<int32_t*>(fake(2)), fake(3),
                               12288, fake(4), fake(5), static_cast<int64_t*>(fake(6)),
                               static_cast<int32_t*>(fake(7)), static_cast<int32_t*>(fake(8)),
                               static_cast<int64_t*>(fake(9)), 256, 256, &s, nullptr) == INV);
  // copy-engine puts
  const void* src[HOCF_MAX_PUTS + 1];
  void* dst[HOCF_MAX_PUTS + 1];
  int64_t bytes[HOCF_MAX_PUTS + 1];
  uint32_t* sig[HOCF_MAX_PUTS + 1];
  for (int i = 0; i <= HOCF_MAX_PUTS; ++i) {
    src[i] = fake(80 + i % 8);
    dst[i] = static_cast<char*>(fake(90)) + (int64_t)i * 8192;
    bytes[i] = 4096;
    sig[i] = fake32(91) + i;
  }
  EXPECT(hocf_dma_put(HOCF_MAX_PUTS + 1, src, dst, bytes, sig, fake32(92), HOCF_ENGINE_DMA, nullptr) == INV);
  EXPECT(hocf_dma_put(2, src, dst, bytes, sig, fake32(92), static_cast<hocf_engine>(7), nullptr) == INV);
  EXPECT(hocf_dma_put(2, src, dst, bytes, sig, nullptr, HOCF_ENGINE_DMA, nullptr) == INV);
  dst[1] = static_cast<char*>(dst[0]) + 16;  // two destinations overlap
  EXPECT(hocf_dma_put(2, src, dst, bytes, sig, fake32(92), HOCF_ENGINE_CU, nullptr) == INV);
  dst[1] = static_cast<char*>(fake(90)) + 8192;
  sig[1] = static_cast<uint32_t*>(dst[0]) + 4;  // a signal word inside a destination
  EXPECT(hocf_dma_put(2, src, dst, bytes, sig, fake32(92), HOCF_ENGINE_DMA, nullptr) == INV);
  EXPECT(hocf_dma_put(0, nullptr, nullptr, nullptr, nullptr, nullptr, HOCF_ENGINE_DMA, nullptr) == HOCF_OK);

  std::printf("abi driver: %d failures\n", fails);
  return fails ? 1 : 0;
}
