// Host sanitizer run of the C ABI's argument validation (test
// infrastructure): tests/test_sanitizers.py compiles the library's host
// code with AddressSanitizer and UndefinedBehaviorSanitizer and links this
// driver, which calls the entry points with arguments that each validation
// rule must reject before anything is enqueued, and the size functions
// with valid and invalid sizes.  No call reaches a launch, so no GPU is
// needed; the sanitizers check the host arithmetic (size products, padded
// limits, workspace planning) for overflow and out-of-bounds accesses.
#include <cstdint>
#include <cstdio>

#include "hsq.h"

static int fails = 0;
static void expect(int got, int want, const char *what) {
  if (got != want) {
    std::fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++fails;
  }
}

int main() {
  const uint16_t *A16 = reinterpret_cast<const uint16_t *>(uintptr_t{0x100000});
  const uint8_t *A8 = reinterpret_cast<const uint8_t *>(uintptr_t{0x100000});
  void *AV = reinterpret_cast<void *>(uintptr_t{0x100000});
  const size_t big = size_t{1} << 40;
  // sizes and limits (M*K, M*N, K*N, padded operand blobs)
  expect(hsq_workspace_bytes(0, 256, 256, 4, 1) == 0, 1, "M = 0");
  expect(hsq_workspace_bytes(1 << 20, 1 << 12, 16, 4, 1) == 0, 1, "M*K >= 2^31");
  expect(hsq_workspace_bytes(1, 1 << 28, 1, 4, 1) == 0, 1, "padded codes >= 2^32");
  expect(hsq_workspace_bytes(4608, 12288, 3072, 4, 1) > 0, 1, "flux down");
  expect(hsq_workspace_bytes_g(2048, 12288, 4096, 32, 2, 128) > 0, 1, "group 128, rank 32");
  expect(hsq_packed_weight_bytes(65536, 32767) > 0, 1, "largest weight");
  expect(hsq_packed_weight_bytes(64, 0) == 0, 1, "N = 0");
  expect(hsq_mlp_workspace_bytes(4608, 3072, 12288, 3072, 4, 0) > 0, 1, "chain, rank-0 down");
  expect(hsq_hessian_workspace_bytes(2048, 4096) >= 0, 1, "hessian");
  expect(hsq_closed_form_l2_workspace_bytes(16384, 16, 32) > 0, 1, "l2");
  // the linear: every rejection before a launch
  expect(hsq_w4a4_lowrank_linear_ex(nullptr, 64, 256, 256, 1, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16, AV,
                                    big, 0, nullptr), HSQ_E_INVAL, "null X");
  expect(hsq_w4a4_lowrank_linear_ex(A16, 64, 100, 256, 1, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16, AV, big,
                                    0, nullptr), HSQ_E_SHAPE, "K % 64");
  expect(hsq_w4a4_lowrank_linear_ex(A16 + 1, 64, 256, 256, 1, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16, AV,
                                    big, 0, nullptr), HSQ_E_ALIGN, "misaligned X");
  expect(hsq_w4a4_lowrank_linear_ex(A16, 64, 256, 256, 1, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16, AV, 16,
                                    0, nullptr), HSQ_E_WORKSPACE, "small workspace");
  expect(hsq_w4a4_lowrank_linear_ex(A16, 32767, 65536, 16, 1, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16, AV,
                                    0, 0, nullptr), HSQ_E_WORKSPACE, "largest token count: sizes pass");
  expect(hsq_w4a4_lowrank_linear_g(A16, 64, 256, 256, 1, 96, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16, AV,
                                   big, 0, nullptr), HSQ_E_INVAL, "group 96");
  expect(hsq_w4a4_lowrank_linear_aq(A16, 64, 256, 256, 1, 64, 7, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16,
                                    AV, big, 0, nullptr), HSQ_E_INVAL, "activation format");
  expect(hsq_w4a4_lowrank_linear_noalloc(A16, 32767, 4096, 16, 1, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16,
                                         nullptr), HSQ_E_SCRATCH, "noalloc beyond the scratch");
  expect(hsq_w4a4_lowrank_linear_noalloc(nullptr, 64, 256, 256, 1, A16, A8, A16, A16, A16, 4, A16, AV, HSQ_BF16,
                                         nullptr), HSQ_E_INVAL, "noalloc null X");
  expect(hsq_w4a4_group_partials(A16, 64, 256, 256, A16, A8, 60, 10, 0, 16, reinterpret_cast<int32_t *>(AV), AV,
                                 big, 0, nullptr), HSQ_E_SHAPE, "window past M");
  expect(hsq_quantize_act(A16, 64, 12352, A16, A16, 4, const_cast<uint8_t *>(A8), const_cast<uint16_t *>(A16),
                          reinterpret_cast<float *>(AV), nullptr), HSQ_E_INVAL, "public quantizer K limit");
  expect(hsq_pack_weights(reinterpret_cast<const int8_t *>(A8), 64, 16, const_cast<uint8_t *>(A8), nullptr,
                          nullptr), HSQ_E_INVAL, "pack null status");
  expect(hsq_mx_lowrank_linear(A16, 64, 256, 256, A16, A8, A16, A16, 4, A16, AV, 3, AV, big, nullptr),
         HSQ_E_INVAL, "mx dtype");
  expect(hsq_w4a4_lowrank_mlp(A16, 64, 256, 512, 256, A16, A8, A16, A16, A16, 4, A16, 5, A16, A8, A16, A16, A16,
                              4, A16, AV, HSQ_BF16, nullptr, AV, big, nullptr), HSQ_E_INVAL, "chain activation");
  expect(hsq_hessian_accumulate(A16, 64, 100, A16, reinterpret_cast<float *>(AV), 0, AV, big, nullptr),
         HSQ_E_SHAPE, "hessian K");
  expect(hsq_deflate_hessian(reinterpret_cast<const float *>(AV), 256, A16, 33,
                             reinterpret_cast<float *>(AV), reinterpret_cast<float *>(AV),
                             reinterpret_cast<double *>(AV), AV, big, nullptr), HSQ_E_INVAL, "deflate rank");
  for (int st = -7; st <= 1; ++st)
    if (!hsq_status_string(st)) ++fails;
  if (fails) return 1;
  std::printf("abi sanitizer run ok\n");
  return 0;
}
