// Host driver for a sanitizer build of the C-ABI validation layer (mxq_api.hip built with
// AddressSanitizer and UndefinedBehaviorSanitizer on its host code).  Every call here must
// be decided on the host: argument errors, empty problems, the host-only scale and
// workspace functions.  No device work is enqueued, so no GPU is needed.  Exit status 0
// when every call returned what it should; the sanitizers abort on the first report.
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/mxq.h"

namespace {

int failures = 0;
int checks = 0;

// fake device pointers: never dereferenced by the validation layer
void* const P16 = reinterpret_cast<void*>(uintptr_t{1} << 20);
void* const P1 = reinterpret_cast<void*>((uintptr_t{1} << 20) + 1);

void expect(const char* what, mxq_status got, bool want_ok) {
  ++checks;
  const bool is_ok = got == MXQ_OK;
  const char* msg = mxq_last_error();
  const bool good = want_ok ? (is_ok && msg[0] == '\0') : (!is_ok && msg[0] != '\0');
  if (!good) {
    ++failures;
    printf("FAIL %s: status %d, message '%s'\n", what, (int)got, msg);
  }
}

const int64_t BIG = INT64_MAX, NEG = INT64_MIN, HUGE_DIM = int64_t{1} << 40;

}  // namespace

int main() {
  auto* u8 = static_cast<uint8_t*>(P16);
  auto* u16 = static_cast<uint16_t*>(P16);
  auto* bad8 = static_cast<uint8_t*>(P1);
  double* d3 = static_cast<double*>(P16);
  float* f1 = static_cast<float*>(P16);

  // quantizers: sizes, pitches and pointers, including values near the int64 limits
  const int64_t dims[][3] = {{-1, 64, 64}, {4, -32, 64}, {4, 48, 64}, {4, 64, 32}, {BIG, 64, 64}, {4, BIG - 31, BIG},
                             {4, 64, BIG}, {4, 64, NEG}, {NEG, 64, 64}, {HUGE_DIM, 64, 64}, {4, 1 << 30, int64_t{1} << 33}};
  for (auto& d : dims) {
    expect("quantize dims", mxq_quantize(P16, MXQ_BF16, d[0], d[1], d[2], u8, 32, u8, 2, nullptr), false);
    expect("quantize_rule dims", mxq_quantize_rule(P16, MXQ_F32, d[0], d[1], d[2], u8, 32, u8, 2, MXQ_SCALE_UOS, nullptr), false);
    expect("hadamard dims", mxq_quantize_hadamard(P16, MXQ_BF16, d[0], d[1], d[2], 64, MXQ_SCALE_OCP, u8, 32, u8, 2, nullptr), false);
    expect("fp8 dims", mxq_quantize_fp8(P16, MXQ_BF16, d[0], d[1], d[2], 1.0f, u8, 64, nullptr), false);
    expect("absmax dims", mxq_absmax(P16, MXQ_BF16, d[0], d[1], d[2], f1, nullptr), false);
  }
  expect("quantize NULL x", mxq_quantize(nullptr, MXQ_BF16, 4, 64, 64, u8, 32, u8, 2, nullptr), false);
  expect("quantize NULL codes", mxq_quantize(P16, MXQ_BF16, 4, 64, 64, nullptr, 32, u8, 2, nullptr), false);
  expect("quantize codes misaligned", mxq_quantize(P16, MXQ_BF16, 4, 64, 64, bad8, 32, u8, 2, nullptr), false);
  expect("quantize ld_codes huge", mxq_quantize(P16, MXQ_BF16, 4, 64, 64, u8, BIG, u8, 2, nullptr), false);
  expect("quantize ld_scales huge", mxq_quantize(P16, MXQ_BF16, 4, 64, 64, u8, 32, u8, BIG, nullptr), false);
  expect("quantize dtype", mxq_quantize(P16, (mxq_dtype)7, 4, 64, 64, u8, 32, u8, 2, nullptr), false);
  expect("quantize rule", mxq_quantize_rule(P16, MXQ_BF16, 4, 64, 64, u8, 32, u8, 2, (mxq_scale_rule)9, nullptr), false);
  expect("hadamard block_n", mxq_quantize_hadamard(P16, MXQ_BF16, 4, 64, 64, 32, MXQ_SCALE_OCP, u8, 32, u8, 2, nullptr), false);
  expect("fp8 inv_scale", mxq_quantize_fp8(P16, MXQ_BF16, 4, 64, 64, NAN, u8, 64, nullptr), false);
  expect("fp8 ld_q huge", mxq_quantize_fp8(P16, MXQ_BF16, 4, 64, 64, 1.0f, u8, BIG, nullptr), false);
  expect("absmax out", mxq_absmax(P16, MXQ_BF16, 4, 64, 64, nullptr, nullptr), false);

  // static FP8 scales (host arithmetic)
  const float good_amax[] = {448.0f, 1.0f, 3e-5f, 7e20f, FLT_MAX, 1e-30f, 6.25e-36f};
  for (float a : good_amax) {
    float s = 0, inv = 0;
    expect("fp8_static_scales", mxq_fp8_static_scales(a, &s, &inv), true);
  }
  const float bad_amax[] = {0.0f, -1.0f, INFINITY, -INFINITY, NAN, 1e-40f, 4e-45f};
  for (float a : bad_amax) {
    float s = 0, inv = 0;
    expect("fp8_static_scales bad", mxq_fp8_static_scales(a, &s, &inv), false);
  }
  expect("fp8_static_scales NULL", mxq_fp8_static_scales(1.0f, nullptr, nullptr), false);

  // GEMMs
  const int64_t gd[][4] = {{-1, 8, 64, 8}, {8, 8, 48, 8}, {8, 8, 64, 4}, {BIG, 8, 64, 8}, {8, BIG, 64, BIG},
                           {8, 8, BIG - 31, 8}, {8, 8, 64, BIG}, {8, 8, 64, NEG}, {NEG, NEG, NEG, NEG},
                           {HUGE_DIM, HUGE_DIM, 1 << 20, HUGE_DIM}, {8, 8, int64_t{1} << 22, 8}};
  for (auto& g : gd) {
    expect("w4a4 dims", mxq_gemm_w4a4(u8, u8, u8, u8, g[0], g[1], g[2], u16, g[3], nullptr), false);
    expect("w4a8 dims", mxq_gemm_w4a8(u8, 1.0f, u8, u8, g[0], g[1], g[2], u16, g[3], nullptr), false);
    expect("bf16 dims", mxq_gemm_bf16(u16, u16, g[0], g[1], g[2], u16, g[3], nullptr), false);
    expect("fused dims", mxq_gemm_w4a4_fused(P16, MXQ_BF16, g[2], u8, u8, g[0], g[1], g[2], MXQ_SCALE_OCP, u16, g[3],
                                             nullptr, 0, nullptr), false);
    (void)mxq_gemm_w4a4_fused_workspace_bytes(g[0], g[1], g[2]);
  }
  expect("w4a4 NULL a", mxq_gemm_w4a4(nullptr, u8, u8, u8, 8, 8, 64, u16, 8, nullptr), false);
  expect("w4a4 misaligned out", mxq_gemm_w4a4(u8, u8, u8, u8, 8, 8, 64, reinterpret_cast<uint16_t*>(bad8), 8, nullptr), false);
  expect("w4a8 scale", mxq_gemm_w4a8(u8, INFINITY, u8, u8, 8, 8, 64, u16, 8, nullptr), false);
  expect("fused ld_a huge", mxq_gemm_w4a4_fused(P16, MXQ_BF16, BIG, u8, u8, 8, 8, 64, MXQ_SCALE_OCP, u16, 8, nullptr, 0,
                                                nullptr), false);
  expect("fused workspace small", mxq_gemm_w4a4_fused(P16, MXQ_BF16, 8192, u8, u8, 8, 1024, 8192, MXQ_SCALE_OCP, u16,
                                                      1024, P16, 16, nullptr), false);
  expect("fused workspace misaligned", mxq_gemm_w4a4_fused(P16, MXQ_BF16, 8192, u8, u8, 8, 1024, 8192, MXQ_SCALE_OCP,
                                                           u16, 1024, P1, size_t{1} << 30, nullptr), false);
  const int64_t wq[][3] = {{BIG, BIG, BIG}, {NEG, 1, 32}, {75600, 5120, 13824}, {1, 1, 32}, {BIG, 5120, 1 << 21}};
  for (auto& q : wq) (void)mxq_gemm_w4a4_fused_workspace_bytes(q[0], q[1], q[2]);
  if (mxq_gemm_w4a4_fused_workspace_bytes(75600, 5120, 13824) != size_t{75600} * 6912 + size_t{75600} * 432) {
    ++failures;
    printf("FAIL fused workspace size\n");
  }

  // SQNR and dequantization
  const int64_t sd[][3] = {{-1, 64, 64}, {4, 60, 64}, {4, 64, 60}, {BIG, 64, 64}, {4, BIG - 7, BIG}, {4, 64, BIG},
                           {NEG, NEG, NEG}, {HUGE_DIM, 64, 64}};
  for (auto& d : sd) {
    expect("sqnr dims", mxq_sqnr(u16, u16, d[0], d[1], d[2], d[2], P16, 1 << 16, d3, nullptr), false);
    expect("sqnr_noalloc dims", mxq_sqnr_noalloc(u16, u16, d[0], d[1], d[2], d[2], d3, nullptr), false);
    expect("dequantize dims", mxq_dequantize(u8, d[2], u8, d[2], d[0], d[1], u16, d[2], nullptr), false);
    expect("dequantize_fp8 dims", mxq_dequantize_fp8(u8, d[2], 1.0f, d[0], d[1], u16, d[2], nullptr), false);
  }
  (void)mxq_sqnr_workspace_bytes(BIG);
  (void)mxq_sqnr_workspace_bytes(NEG);
  expect("sqnr workspace", mxq_sqnr(u16, u16, 4, 64, 64, 64, nullptr, 0, d3, nullptr), false);
  expect("sqnr out3", mxq_sqnr(u16, u16, 4, 64, 64, 64, P16, 1 << 16, nullptr, nullptr), false);
  expect("dequantize NULL", mxq_dequantize(nullptr, 32, u8, 2, 4, 64, u16, 64, nullptr), false);
  expect("dequantize_fp8 scale", mxq_dequantize_fp8(u8, 64, NAN, 4, 64, u16, 64, nullptr), false);

  // the register-only MFMA loop's arguments
  expect("ceiling mode", mxq_mfma_ceiling((mxq_gemm_mode)5, P16, u8, P16, u8, 8, 8, 64, 4, 1, f1, nullptr), false);
  expect("ceiling waves", mxq_mfma_ceiling(MXQ_GEMM_W4A4, P16, u8, P16, u8, 8, 8, 64, BIG, 1, f1, nullptr), false);
  expect("ceiling dims", mxq_mfma_ceiling(MXQ_GEMM_BF16, P16, nullptr, P16, nullptr, BIG, BIG, BIG, 4, 1, f1, nullptr), false);

  // empty problems are valid and touch nothing
  expect("quantize empty", mxq_quantize(nullptr, MXQ_BF16, 0, 64, 64, nullptr, 32, nullptr, 2, nullptr), true);
  expect("w4a4 empty", mxq_gemm_w4a4(nullptr, nullptr, nullptr, nullptr, 0, 8, 64, nullptr, 8, nullptr), true);
  expect("fused empty", mxq_gemm_w4a4_fused(nullptr, MXQ_BF16, 64, nullptr, nullptr, 0, 8, 64, MXQ_SCALE_OCP, nullptr,
                                            8, nullptr, 0, nullptr), true);
  expect("dequantize empty", mxq_dequantize(nullptr, 32, nullptr, 2, 0, 64, nullptr, 64, nullptr), true);

  if (mxq_abi_version() != MXQ_ABI_VERSION) {
    ++failures;
    printf("FAIL abi version\n");
  }
  printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
