// Host-sanitizer (AddressSanitizer + UndefinedBehaviorSanitizer) check of
// libsnip's argument validation and sizing: every entry point of
// include/snip.h is called with rejected arguments (NULL pointers, bad
// shapes, misaligned pointers, unknown formats, short workspaces, layers too
// large for the static scratch) and every sizing helper over a sweep of
// shapes. None of these calls reaches the GPU (validation precedes any HIP
// call), so this runs on a machine without one. Built with the library's
// host code instrumented (sub_byte_mixed_amd/build.py build_asan_check);
// exit status 0 iff every status code is the documented one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/snip.h"

static int g_fail = 0;
#define EXPECT(call, code)                                                                 \
  do {                                                                                     \
    const int rc_ = (call);                                                                \
    if (rc_ != (code)) {                                                                   \
      std::printf("FAIL line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, \
                  (code), snip_last_error());                                             \
      ++g_fail;                                                                            \
    } else if ((code) != SNIP_OK && std::strlen(snip_last_error()) == 0) {                \
      std::printf("FAIL line %d: %s: no error message\n", __LINE__, #call);                \
      ++g_fail;                                                                            \
    }                                                                                      \
  } while (0)

int main() {
  // fake, 256-aligned device addresses: never dereferenced by rejected calls
  void* const P = reinterpret_cast<void*>(uintptr_t(0x7F0000000000ull));
  void* const P2 = reinterpret_cast<void*>(uintptr_t(0x7F0000100000ull));
  void* const Pm = reinterpret_cast<void*>(uintptr_t(0x7F0000000004ull));   // misaligned
  float* const F = static_cast<float*>(P);
  snip_stats* const ST = static_cast<snip_stats*>(P2);
  int32_t* const E = static_cast<int32_t*>(P2);

  // ---- sizing over a sweep of shapes (every path of plan_gemm)
  const int64_t dims[] = {1, 15, 16, 17, 128, 240, 256, 1000, 1024, 2048, 4096, 5632, 28672};
  size_t acc = 0;
  for (int64_t M : dims)
    for (int64_t N : dims)
      for (int64_t Kk : {int64_t(128), int64_t(256), int64_t(2048), int64_t(8192)})
        for (int f = -1; f <= 8; ++f) {
          acc += snip_qgemm_workspace(M, N, Kk, f) + snip_linear_fwd_workspace(M, Kk, N, f) +
                 snip_linear_bwd_workspace(M, Kk, N, f, f) + snip_quantize_dual_workspace(M, N, f) +
                 snip_linear_fwd_save_workspace(M, Kk, N, f) + snip_linear_bwd_saved_workspace(M, Kk, N, f) +
                 snip_qgemm_qout_workspace(M, N, Kk, f) + snip_quantize_workspace(M, N, SNIP_ROWWISE, f);
          for (int op = -1; op <= 8; ++op) acc += snip_workspace_size(op, M, N, Kk, f);
          for (int part = -1; part <= 2; ++part) acc += (size_t)snip_qtensor_bytes(f, M, Kk, part);
        }
  if (snip_qgemm_workspace(0, 16, 128, SNIP_NVFP4) != 0 || snip_workspace_size(99, 1, 1, 1, 1) != 0) ++g_fail;

  snip_qtensor q{SNIP_NVFP4, 0, 256, 512, P, P2, E};
  snip_qtensor qk{SNIP_NVFP4, 0, 512, 512, P, P2, E};
  snip_qtensor bad{9, 0, 256, 512, P, P2, E};
  snip_qtensor mis{SNIP_NVFP4, 0, 256, 512, Pm, P2, E};

  // ---- snip_quantize
  EXPECT(snip_quantize(nullptr, 256, 512, 512, SNIP_ROWWISE, SNIP_NVFP4, SNIP_RNE, 0, 0, nullptr, &q, nullptr, P,
                       1 << 20, nullptr), SNIP_E_NULL);
  EXPECT(snip_quantize(P, 256, 500, 512, SNIP_ROWWISE, SNIP_NVFP4, SNIP_RNE, 0, 0, nullptr, &q, nullptr, P, 1 << 20,
                       nullptr), SNIP_E_SHAPE);
  EXPECT(snip_quantize(P, 256, 512, 512, SNIP_ROWWISE, 12, SNIP_RNE, 0, 0, nullptr, &q, nullptr, P, 1 << 20, nullptr),
         SNIP_E_FORMAT);
  EXPECT(snip_quantize(P, 256, 512, 512, 7, SNIP_NVFP4, SNIP_RNE, 0, 0, nullptr, &q, nullptr, P, 1 << 20, nullptr),
         SNIP_E_FORMAT);
  EXPECT(snip_quantize(Pm, 256, 512, 512, SNIP_ROWWISE, SNIP_NVFP4, SNIP_RNE, 0, 0, nullptr, &q, nullptr, P, 1 << 20,
                       nullptr), SNIP_E_ALIGN);
  EXPECT(snip_quantize(P, 256, 512, 512, SNIP_ROWWISE, SNIP_NVFP4, SNIP_RNE, 0, 0, nullptr, &q, nullptr, P, 8,
                       nullptr), SNIP_E_WORKSPACE);
  EXPECT(snip_quantize(P, 256, 512, 512, SNIP_ROWWISE, SNIP_NVFP4, SNIP_RNE, 0, 0, nullptr, &mis, nullptr, P,
                       1 << 20, nullptr), SNIP_E_ALIGN);
  EXPECT(snip_quantize(P, 256, 512, 512, SNIP_ROWWISE, SNIP_NVFP4, SNIP_RNE, 0, 0, nullptr, &bad, nullptr, P,
                       1 << 20, nullptr), SNIP_E_FORMAT);

  // ---- snip_qgemm / snip_qgemm_qout
  EXPECT(snip_qgemm(nullptr, &q, F, 256, nullptr, 0, nullptr), SNIP_E_NULL);
  EXPECT(snip_qgemm(&q, &qk, F, 100, nullptr, 0, nullptr), SNIP_E_SHAPE);
  snip_qtensor qm{SNIP_MXFP4, 0, 256, 512, P, P2, E};
  EXPECT(snip_qgemm(&q, &qm, F, 512, nullptr, 0, nullptr), SNIP_E_FORMAT);
  snip_qtensor qv{SNIP_FP4_BF16_B16, 0, 256, 512, P, P2, E};
  EXPECT(snip_qgemm(&qv, &qv, F, 256, nullptr, 0, nullptr), SNIP_E_FORMAT);
  snip_qtensor q100{SNIP_NVFP4, 0, 256, 400, P, P2, E};
  EXPECT(snip_qgemm(&q100, &q100, F, 256, nullptr, 0, nullptr), SNIP_E_SHAPE);
  snip_qtensor qo{SNIP_NVFP4, 0, 256, 512, P, P2, E};
  EXPECT(snip_qgemm_qout(&q, &qk, F, 512, SNIP_RNE, 0, 0, nullptr, &qo, nullptr, P, 1 << 20, nullptr), SNIP_E_NULL);
  EXPECT(snip_qgemm_qout(&qm, &qm, F, 512, SNIP_RNE, 0, 0, F, &qo, nullptr, P, 1 << 20, nullptr), SNIP_E_FORMAT);
  EXPECT(snip_qgemm_qout(&q, &qk, F, 514, SNIP_RNE, 0, 0, F, &qo, nullptr, P, 1 << 20, nullptr), SNIP_E_SHAPE);
  EXPECT(snip_qgemm_qout(&q, &qk, F, 512, 5, 0, 0, F, &qo, nullptr, P, 1 << 20, nullptr), SNIP_E_FORMAT);
  EXPECT(snip_qgemm_qout(&q, &qk, F, 512, SNIP_SR, 0, 0, F, &qo, nullptr, P, 0, nullptr), SNIP_E_WORKSPACE);

  // ---- layer calls
  EXPECT(snip_linear_fwd(nullptr, P, 256, 512, 512, SNIP_NVFP4, 0, 0, F, nullptr, P, 1 << 30, nullptr), SNIP_E_NULL);
  EXPECT(snip_linear_fwd(P, P, 256, 500, 512, SNIP_NVFP4, 0, 0, F, nullptr, P, 1 << 30, nullptr), SNIP_E_SHAPE);
  EXPECT(snip_linear_fwd(P, P, 256, 512, 512, SNIP_FP4_E8M0_B16, 0, 0, F, nullptr, P, 1 << 30, nullptr),
         SNIP_E_FORMAT);
  EXPECT(snip_linear_fwd(P, P, 256, 512, 512, SNIP_NVFP4, 0, 0, F, nullptr, P, 16, nullptr), SNIP_E_WORKSPACE);
  EXPECT(snip_linear_bwd(P, P, nullptr, 256, 512, 512, SNIP_NVFP4, SNIP_NVFP4, 0, 0, nullptr, F, F, nullptr, P,
                         1 << 30, nullptr), SNIP_E_NULL);
  EXPECT(snip_linear_bwd(P, P, P, 200, 512, 512, SNIP_NVFP4, SNIP_NVFP4, 0, 0, nullptr, F, F, nullptr, P, 1 << 30,
                         nullptr), SNIP_E_SHAPE);
  EXPECT(snip_linear_bwd(P, P, P, 256, 512, 512, SNIP_NVFP4, 9, 0, 0, nullptr, F, F, nullptr, P, 1 << 30, nullptr),
         SNIP_E_FORMAT);
  EXPECT(snip_linear_bwd(P, P, P, 256, 512, 512, SNIP_NVFP4, SNIP_NVFP4, 0, 0, nullptr, F, F, nullptr, P, 64,
                         nullptr), SNIP_E_WORKSPACE);
  snip_qtensor q2{SNIP_NVFP4, 0, 256, 512, P, P2, E};
  snip_qtensor qr{SNIP_NVFP4, 0, 512, 512, P, P2, E};
  EXPECT(snip_quantize_dual(P, 256, 512, 512, SNIP_BF16, SNIP_RNE, SNIP_SR, 0, 0, 1, nullptr, &q2, &qr, nullptr, P,
                            1 << 20, nullptr), SNIP_E_FORMAT);
  EXPECT(snip_quantize_dual(P, 256, 512, 512, SNIP_NVFP4, SNIP_RNE, SNIP_SR, 0, 0, 1, nullptr, &q2, &q2, nullptr, P,
                            1 << 20, nullptr), SNIP_E_SHAPE);
  snip_qtensor wt{SNIP_NVFP4, 0, 512, 512, P, P2, E};
  snip_qtensor xt{SNIP_NVFP4, 0, 512, 256, P, P2, E};
  EXPECT(snip_linear_fwd_save(P, P, 256, 512, 512, SNIP_NVFP4, 0, 0, nullptr, nullptr, F, &wt, &xt, nullptr, P, 64,
                              nullptr), SNIP_E_WORKSPACE);
  EXPECT(snip_linear_fwd_save(P, P, 256, 512, 512, SNIP_NVFP4, 0, 0, nullptr, nullptr, F, &xt, &wt, nullptr, P,
                              1 << 30, nullptr), SNIP_E_SHAPE);
  EXPECT(snip_linear_bwd_saved(P, &wt, &xt, 256, 512, 512, 0, 0, nullptr, F, F, nullptr, P, 64, nullptr),
         SNIP_E_WORKSPACE);
  EXPECT(snip_linear_bwd_saved(nullptr, &wt, &xt, 256, 512, 512, 0, 0, nullptr, F, F, nullptr, P, 1 << 30, nullptr),
         SNIP_E_NULL);
  // the allocation-free forward: a layer beyond the static scratch, and bad arguments
  snip_qtensor wt7{SNIP_NVFP4, 0, 4096, 11008, P, P2, E};
  snip_qtensor xt7{SNIP_NVFP4, 0, 4096, 8192, P, P2, E};
  EXPECT(snip_linear_fwd_save_noalloc(P, P, 8192, 4096, 11008, SNIP_NVFP4, 0, 0, nullptr, nullptr, F, &wt7, &xt7,
                                      nullptr, nullptr), SNIP_E_WORKSPACE);
  EXPECT(snip_linear_fwd_save_noalloc(P, P, 256, 512, 512, SNIP_BF16, 0, 0, nullptr, nullptr, F, &wt, &xt, nullptr,
                                      nullptr), SNIP_E_FORMAT);
  EXPECT(snip_linear_fwd_save_noalloc(P, P, 256, 512, 512, SNIP_NVFP4, 0, 0, nullptr, nullptr, nullptr, &wt, &xt,
                                      nullptr, nullptr), SNIP_E_NULL);

  // ---- statistics report and timing
  snip_tensor_report rep[2];
  EXPECT(snip_layer_stats(nullptr, 1, rep, nullptr), SNIP_E_NULL);
  EXPECT(snip_layer_stats(ST, 0, rep, nullptr), SNIP_E_SHAPE);
  EXPECT(snip_layer_stats(ST, 100000, rep, nullptr), SNIP_E_SHAPE);
  EXPECT(snip_timing_start(0), SNIP_E_SHAPE);
  EXPECT(snip_timing_read(nullptr, 0, nullptr), SNIP_E_FORMAT);
  if (snip_version() <= 0) ++g_fail;

  std::printf("{\"failures\": %d, \"sized\": %zu}\n", g_fail, acc);
  return g_fail ? 1 : 0;
}
