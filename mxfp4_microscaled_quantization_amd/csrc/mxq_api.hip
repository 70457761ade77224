// C ABI of libmxq: argument validation, error reporting and dispatch to the gfx950
// launchers.  Every check runs before anything is enqueued, so an error return means the
// stream was not touched.  The only mutable state is the thread-local error message.
#include <float.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "../../include/mxq.h"
#include "mxq_internal.hpp"

namespace {

thread_local std::string g_error;

mxq_status fail(mxq_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

mxq_status ok() {
  g_error.clear();
  return MXQ_OK;
}

mxq_status hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(MXQ_ERR_HIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Row pitches (elements or bytes) are below 2^32, dimensions below 2^31: every product the
// checks and the launchers form then stays inside int64.
constexpr int64_t kMaxPitch = ((int64_t)1 << 32) - 1;
constexpr int64_t kMaxDim = 0x7FFFFFFF;
bool pitch_ok(int64_t ld) { return ld <= kMaxPitch; }

int dtype_bytes(mxq_dtype dt) {
  switch (dt) {
    case MXQ_F32: return 4;
    case MXQ_BF16: return 2;
    default: return 0;   // unknown: rejected by the callers
  }
}

// Shared checks for a rows x cols input of dtype dt with pitch ld (elements).
mxq_status check_input(const char* fn, const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ld,
                       int64_t col_multiple) {
  if (dtype_bytes(dt) == 0) return fail(MXQ_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dt);
  if (rows < 0 || cols < 0) return fail(MXQ_ERR_INVALID_ARG, "%s: negative size (%lld x %lld)", fn, (long long)rows, (long long)cols);
  if (cols % col_multiple != 0)
    return fail(MXQ_ERR_INVALID_ARG, "%s: cols (%lld) must be a multiple of %lld", fn, (long long)cols,
                (long long)col_multiple);
  if (ld < cols) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_x (%lld) < cols (%lld)", fn, (long long)ld, (long long)cols);
  if (rows > kMaxDim || cols > kMaxDim) return fail(MXQ_ERR_INVALID_ARG, "%s: dimension exceeds 2^31-1", fn);
  if (!pitch_ok(ld)) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_x (%lld) must be below 2^32", fn, (long long)ld);
  if (rows > 0 && cols > 0) {
    if (!x) return fail(MXQ_ERR_INVALID_ARG, "%s: x is NULL", fn);
    if (!aligned(x, 16) || (ld * dtype_bytes(dt)) % 16 != 0)
      return fail(MXQ_ERR_INVALID_ARG, "%s: x base and row pitch must be 16-byte aligned", fn);
  }
  if ((rows * (cols / 8 > 0 ? cols / 8 : 1)) >= ((int64_t)1 << 32))
    return fail(MXQ_ERR_INVALID_ARG, "%s: tensor too large (more than 2^35 elements)", fn);
  return MXQ_OK;
}

mxq_status check_gemm(const char* fn, int64_t M, int64_t N, int64_t K, const void* out, int64_t ld_out) {
  if (M < 0 || N < 0 || K < 0)
    return fail(MXQ_ERR_INVALID_ARG, "%s: negative size (M=%lld N=%lld K=%lld)", fn, (long long)M, (long long)N,
                (long long)K);
  if (K % 32 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: K (%lld) must be a multiple of 32", fn, (long long)K);
  if (M > (int64_t)0x7FFFFFFF - 256 || N > (int64_t)0x7FFFFFFF - 256 || K > ((int64_t)1 << 21))
    return fail(MXQ_ERR_INVALID_ARG, "%s: dimension too large", fn);
  if (ld_out < N) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_out (%lld) < N (%lld)", fn, (long long)ld_out, (long long)N);
  if (!pitch_ok(ld_out)) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_out (%lld) must be below 2^32", fn, (long long)ld_out);
  if (M > 0 && N > 0) {
    if (!out) return fail(MXQ_ERR_INVALID_ARG, "%s: out is NULL", fn);
    if (!aligned(out, 2)) return fail(MXQ_ERR_INVALID_ARG, "%s: out must be 2-byte aligned", fn);
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (tiles > 0x7FFFFFFF) return fail(MXQ_ERR_INVALID_ARG, "%s: problem too large", fn);
  }
  return MXQ_OK;
}

mxq_status check_operand(const char* fn, const char* name, const void* p, int64_t rows, int64_t K, int align) {
  if (rows > 0 && K > 0) {
    if (!p) return fail(MXQ_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
    if (!aligned(p, (uintptr_t)align)) return fail(MXQ_ERR_INVALID_ARG, "%s: %s must be %d-byte aligned", fn, name, align);
  }
  return MXQ_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int mxq_abi_version(void) { return MXQ_ABI_VERSION; }

const char* mxq_last_error(void) { return g_error.c_str(); }

mxq_status mxq_quantize_rule(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                             int64_t ld_codes, uint8_t* scales, int64_t ld_scales, mxq_scale_rule rule, void* stream) {
  const char* fn = "mxq_quantize";
  if (rule != MXQ_SCALE_OCP && rule != MXQ_SCALE_UOS)
    return fail(MXQ_ERR_UNSUPPORTED, "%s: unknown scale rule %d", fn, (int)rule);
  mxq_status st = check_input(fn, x, dt, rows, cols, ld_x, 32);
  if (st != MXQ_OK) return st;
  if (ld_codes < cols / 2) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_codes (%lld) < cols/2", fn, (long long)ld_codes);
  if (ld_scales < cols / 32) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_scales (%lld) < cols/32", fn, (long long)ld_scales);
  if (!pitch_ok(ld_codes) || !pitch_ok(ld_scales)) return fail(MXQ_ERR_INVALID_ARG, "%s: pitch must be below 2^32", fn);
  if (rows > 0 && cols > 0) {
    if (!codes || !scales) return fail(MXQ_ERR_INVALID_ARG, "%s: codes/scales is NULL", fn);
    if (!aligned(codes, 16) || ld_codes % 16 != 0)
      return fail(MXQ_ERR_INVALID_ARG, "%s: codes base and ld_codes must be multiples of 16 bytes", fn);
  }
  return hip_status(fn, mxq::launch_quantize_mxfp4(x, dt == MXQ_F32, rows, cols, ld_x, codes, ld_codes, scales,
                                                   ld_scales, rule == MXQ_SCALE_UOS, as_stream(stream)));
}

mxq_status mxq_quantize(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                        int64_t ld_codes, uint8_t* scales, int64_t ld_scales, void* stream) {
  return mxq_quantize_rule(x, dt, rows, cols, ld_x, codes, ld_codes, scales, ld_scales, MXQ_SCALE_OCP, stream);
}

mxq_status mxq_quantize_hadamard(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, int block_n,
                                 mxq_scale_rule rule, uint8_t* codes, int64_t ld_codes, uint8_t* scales,
                                 int64_t ld_scales, void* stream) {
  const char* fn = "mxq_quantize_hadamard";
  if (block_n != 16 && block_n != 64 && block_n != 256)
    return fail(MXQ_ERR_UNSUPPORTED, "%s: block_n must be 16, 64 or 256 (got %d)", fn, block_n);
  if (rule != MXQ_SCALE_OCP && rule != MXQ_SCALE_UOS)
    return fail(MXQ_ERR_UNSUPPORTED, "%s: unknown scale rule %d", fn, (int)rule);
  mxq_status st = check_input(fn, x, dt, rows, cols, ld_x, 32);
  if (st != MXQ_OK) return st;
  if (cols % block_n != 0)
    return fail(MXQ_ERR_INVALID_ARG, "%s: cols (%lld) must be a multiple of block_n (%d)", fn, (long long)cols, block_n);
  if (ld_codes < cols / 2) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_codes (%lld) < cols/2", fn, (long long)ld_codes);
  if (ld_scales < cols / 32) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_scales (%lld) < cols/32", fn, (long long)ld_scales);
  if (!pitch_ok(ld_codes) || !pitch_ok(ld_scales)) return fail(MXQ_ERR_INVALID_ARG, "%s: pitch must be below 2^32", fn);
  if (rows > 0 && cols > 0) {
    if (!codes || !scales) return fail(MXQ_ERR_INVALID_ARG, "%s: codes/scales is NULL", fn);
    if (!aligned(codes, 16) || ld_codes % 16 != 0)
      return fail(MXQ_ERR_INVALID_ARG, "%s: codes base and ld_codes must be multiples of 16 bytes", fn);
  }
  return hip_status(fn, mxq::launch_quantize_mxfp4_rotated(x, dt == MXQ_F32, rows, cols, ld_x, block_n, codes, ld_codes,
                                                           scales, ld_scales, rule == MXQ_SCALE_UOS, as_stream(stream)));
}

mxq_status mxq_quantize_fp8(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, float inv_scale,
                            uint8_t* q, int64_t ld_q, void* stream) {
  const char* fn = "mxq_quantize_fp8";
  mxq_status st = check_input(fn, x, dt, rows, cols, ld_x, 16);
  if (st != MXQ_OK) return st;
  if (!(inv_scale > 0.0f) || !(inv_scale < __builtin_inff()))
    return fail(MXQ_ERR_INVALID_ARG, "%s: inv_scale must be finite and > 0", fn);
  if (ld_q < cols) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_q (%lld) < cols", fn, (long long)ld_q);
  if (!pitch_ok(ld_q)) return fail(MXQ_ERR_INVALID_ARG, "%s: ld_q (%lld) must be below 2^32", fn, (long long)ld_q);
  if (rows > 0 && cols > 0) {
    if (!q) return fail(MXQ_ERR_INVALID_ARG, "%s: q is NULL", fn);
    if (!aligned(q, 16) || ld_q % 16 != 0)
      return fail(MXQ_ERR_INVALID_ARG, "%s: q base and ld_q must be multiples of 16 bytes", fn);
  }
  return hip_status(fn, mxq::launch_quantize_fp8(x, dt == MXQ_F32, rows, cols, ld_x, inv_scale, q, ld_q,
                                                 as_stream(stream)));
}

mxq_status mxq_fp8_static_scales(float amax, float* s_a, float* inv_s) {
  const char* fn = "mxq_fp8_static_scales";
  if (!s_a || !inv_s) return fail(MXQ_ERR_INVALID_ARG, "%s: s_a/inv_s is NULL", fn);
  if (!(amax > 0.0f) || !(amax <= FLT_MAX))
    return fail(MXQ_ERR_INVALID_ARG, "%s: amax must be finite and > 0 (got %g)", fn, (double)amax);
  // IEEE binary32 division rounds the exact quotient to nearest even: fl32(amax / 448)
  // and fl32(448 / amax)
  const float sa = amax / 448.0f;
  const float inv = 448.0f / amax;
  if (!(inv <= FLT_MAX))
    return fail(MXQ_ERR_INVALID_ARG, "%s: amax (%g) too small: 448 / amax overflows binary32", fn, (double)amax);
  *s_a = sa;
  *inv_s = inv;
  return ok();
}

mxq_status mxq_absmax(const void* x, mxq_dtype dt, int64_t rows, int64_t cols, int64_t ld_x, float* out,
                      void* stream) {
  const char* fn = "mxq_absmax";
  mxq_status st = check_input(fn, x, dt, rows, cols, ld_x, 8);
  if (st != MXQ_OK) return st;
  if (!out || !aligned(out, 4)) return fail(MXQ_ERR_INVALID_ARG, "%s: out must be a non-NULL 4-byte aligned pointer", fn);
  return hip_status(fn, mxq::launch_absmax(x, dt == MXQ_F32, rows, cols, ld_x, out, as_stream(stream)));
}

mxq_status mxq_gemm_w4a4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* w_codes,
                         const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, uint16_t* out_bf16,
                         int64_t ld_out, void* stream) {
  const char* fn = "mxq_gemm_w4a4";
  mxq_status st = check_gemm(fn, M, N, K, out_bf16, ld_out);
  if (st != MXQ_OK) return st;
  if (M > 0 && N > 0) {
    if ((st = check_operand(fn, "a_codes", a_codes, M, K, 16)) != MXQ_OK) return st;
    if ((st = check_operand(fn, "a_scales", a_scales, M, K, 1)) != MXQ_OK) return st;
    if ((st = check_operand(fn, "w_codes", w_codes, N, K, 16)) != MXQ_OK) return st;
    if ((st = check_operand(fn, "w_scales", w_scales, N, K, 1)) != MXQ_OK) return st;
  }
  return hip_status(fn, mxq::launch_gemm(mxq::GEMM_W4A4, a_codes, a_scales, w_codes, w_scales, 1.0f, M, N, K,
                                         out_bf16, ld_out, as_stream(stream)));
}

// Break-even of the fused W4A4 kernel: it quantizes every activation tile once per
// 256-column output tile, so its cost grows with N, while quantization in a pass of its
// own is paid once.  Measured on MI355X (M = 57344 and 75600): fused is the faster up to
// 3 column tiles (N <= 768) for K >= 8192 (K = 12288: 0.99 of the separate pair at N = 768,
// 1.05 at 1024; K = 13824: 0.96 and 1.02) and up to 1 tile for K = 3072 (0.96 at N = 256,
// 1.04 at 512).
int64_t fused_max_col_tiles(int64_t K) { return K >= 8192 ? 3 : 1; }
int64_t round16(int64_t v) { return (v + 15) / 16 * 16; }

size_t mxq_gemm_w4a4_fused_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 32 != 0) return 0;
  if (M > kMaxDim || N > kMaxDim || K > ((int64_t)1 << 21)) return 0;   // a shape the GEMM rejects
  if ((N + 255) / 256 <= fused_max_col_tiles(K)) return 0;
  return (size_t)(round16(M * (K / 2)) + M * (K / 32));
}

mxq_status mxq_gemm_w4a4_fused(const void* a, mxq_dtype dt, int64_t ld_a, const uint8_t* w_codes,
                               const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, mxq_scale_rule rule,
                               uint16_t* out_bf16, int64_t ld_out, void* workspace, size_t ws_bytes,
                               void* stream) {
  const char* fn = "mxq_gemm_w4a4_fused";
  if (rule != MXQ_SCALE_OCP && rule != MXQ_SCALE_UOS)
    return fail(MXQ_ERR_UNSUPPORTED, "%s: unknown scale rule %d", fn, (int)rule);
  if (dtype_bytes(dt) == 0) return fail(MXQ_ERR_UNSUPPORTED, "%s: unknown dtype %d", fn, (int)dt);
  mxq_status st = check_gemm(fn, M, N, K, out_bf16, ld_out);
  if (st != MXQ_OK) return st;
  if (M > 0 && N > 0) {
    if ((st = check_input(fn, a, dt, M, K, ld_a, 32)) != MXQ_OK) return st;
    if (ld_a * dtype_bytes(dt) * 256 >= ((int64_t)1 << 31))
      return fail(MXQ_ERR_INVALID_ARG, "%s: row pitch too large (256 * ld_a * element size must be below 2^31 bytes)",
                  fn);
    if ((st = check_operand(fn, "w_codes", w_codes, N, K, 16)) != MXQ_OK) return st;
    if ((st = check_operand(fn, "w_scales", w_scales, N, K, 1)) != MXQ_OK) return st;
    if (K > 0 && !a) return fail(MXQ_ERR_INVALID_ARG, "%s: a is NULL", fn);
  }
  const size_t need = mxq_gemm_w4a4_fused_workspace_bytes(M, N, K);
  if (workspace && need > 0) {
    // past the break-even: quantize into the workspace, then the W4A4 GEMM (the same bits)
    if (!aligned(workspace, 16) || ws_bytes < need)
      return fail(MXQ_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned and at least %zu bytes (got %zu)", fn,
                  need, ws_bytes);
    uint8_t* codes = static_cast<uint8_t*>(workspace);
    uint8_t* scales = codes + round16(M * (K / 2));
    hipError_t e = mxq::launch_quantize_mxfp4(a, dt == MXQ_F32, M, K, ld_a, codes, K / 2, scales, K / 32,
                                              rule == MXQ_SCALE_UOS, as_stream(stream));
    if (e != hipSuccess) return hip_status(fn, e);
    return hip_status(fn, mxq::launch_gemm(mxq::GEMM_W4A4, codes, scales, w_codes, w_scales, 1.0f, M, N, K, out_bf16,
                                           ld_out, as_stream(stream)));
  }
  return hip_status(fn, mxq::launch_gemm_w4a4_fused(a, dt == MXQ_F32, ld_a, w_codes, w_scales, M, N, K,
                                                    rule == MXQ_SCALE_UOS, out_bf16, ld_out, as_stream(stream)));
}

mxq_status mxq_gemm_w4a8(const uint8_t* a_fp8, float a_scale, const uint8_t* w_codes, const uint8_t* w_scales,
                         int64_t M, int64_t N, int64_t K, uint16_t* out_bf16, int64_t ld_out, void* stream) {
  const char* fn = "mxq_gemm_w4a8";
  mxq_status st = check_gemm(fn, M, N, K, out_bf16, ld_out);
  if (st != MXQ_OK) return st;
  if (!(a_scale == a_scale) || a_scale == __builtin_inff() || a_scale == -__builtin_inff())
    return fail(MXQ_ERR_INVALID_ARG, "%s: a_scale must be finite", fn);
  if (M > 0 && N > 0) {
    if ((st = check_operand(fn, "a_fp8", a_fp8, M, K, 16)) != MXQ_OK) return st;
    if ((st = check_operand(fn, "w_codes", w_codes, N, K, 16)) != MXQ_OK) return st;
    if ((st = check_operand(fn, "w_scales", w_scales, N, K, 1)) != MXQ_OK) return st;
  }
  return hip_status(fn, mxq::launch_gemm(mxq::GEMM_W4A8, a_fp8, nullptr, w_codes, w_scales, a_scale, M, N, K,
                                         out_bf16, ld_out, as_stream(stream)));
}

mxq_status mxq_gemm_bf16(const uint16_t* a, const uint16_t* w, int64_t M, int64_t N, int64_t K, uint16_t* out,
                         int64_t ld_out, void* stream) {
  const char* fn = "mxq_gemm_bf16";
  mxq_status st = check_gemm(fn, M, N, K, out, ld_out);
  if (st != MXQ_OK) return st;
  if (M > 0 && N > 0) {
    if ((st = check_operand(fn, "a", a, M, K, 16)) != MXQ_OK) return st;
    if ((st = check_operand(fn, "w", w, N, K, 16)) != MXQ_OK) return st;
  }
  return hip_status(fn, mxq::launch_gemm(mxq::GEMM_BF16, a, nullptr, w, nullptr, 1.0f, M, N, K, out, ld_out,
                                         as_stream(stream)));
}

size_t mxq_sqnr_workspace_bytes(int64_t n_elements) { return mxq::sqnr_workspace_bytes(n_elements); }

mxq_status mxq_sqnr(const uint16_t* ref, const uint16_t* test, int64_t rows, int64_t cols, int64_t ld_ref,
                    int64_t ld_test, void* workspace, size_t ws_bytes, double* out3, void* stream) {
  const char* fn = "mxq_sqnr";
  if (rows < 0 || cols < 0) return fail(MXQ_ERR_INVALID_ARG, "%s: negative size", fn);
  if (cols % 8 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: cols (%lld) must be a multiple of 8", fn, (long long)cols);
  if (ld_ref < cols || ld_test < cols) return fail(MXQ_ERR_INVALID_ARG, "%s: pitch below cols", fn);
  if (ld_ref % 8 != 0 || ld_test % 8 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: pitches must be multiples of 8", fn);
  if (rows > kMaxDim || cols > kMaxDim || !pitch_ok(ld_ref) || !pitch_ok(ld_test) ||
      rows * (cols / 8) >= ((int64_t)1 << 32))
    return fail(MXQ_ERR_INVALID_ARG, "%s: tensor too large", fn);
  if (!out3 || !aligned(out3, 8)) return fail(MXQ_ERR_INVALID_ARG, "%s: out3 must be a non-NULL 8-byte aligned pointer", fn);
  if (!workspace || !aligned(workspace, 8) || ws_bytes < mxq::sqnr_workspace_bytes(rows * cols))
    return fail(MXQ_ERR_INVALID_ARG, "%s: workspace missing, misaligned or smaller than %zu bytes", fn,
                mxq::sqnr_workspace_bytes(rows * cols));
  if (rows > 0 && cols > 0) {
    if (!ref || !test) return fail(MXQ_ERR_INVALID_ARG, "%s: ref/test is NULL", fn);
    if (!aligned(ref, 16) || !aligned(test, 16)) return fail(MXQ_ERR_INVALID_ARG, "%s: ref/test must be 16-byte aligned", fn);
  }
  return hip_status(fn, mxq::launch_sqnr(ref, test, rows, cols, ld_ref, ld_test, workspace, out3, as_stream(stream)));
}

mxq_status mxq_sqnr_noalloc(const uint16_t* ref, const uint16_t* test, int64_t rows, int64_t cols, int64_t ld_ref,
                            int64_t ld_test, double* out3, void* stream) {
  const char* fn = "mxq_sqnr_noalloc";
  if (rows < 0 || cols < 0) return fail(MXQ_ERR_INVALID_ARG, "%s: negative size", fn);
  if (cols % 8 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: cols (%lld) must be a multiple of 8", fn, (long long)cols);
  if (ld_ref < cols || ld_test < cols) return fail(MXQ_ERR_INVALID_ARG, "%s: pitch below cols", fn);
  if (ld_ref % 8 != 0 || ld_test % 8 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: pitches must be multiples of 8", fn);
  if (rows > kMaxDim || cols > kMaxDim || !pitch_ok(ld_ref) || !pitch_ok(ld_test) ||
      rows * (cols / 8) >= ((int64_t)1 << 32))
    return fail(MXQ_ERR_INVALID_ARG, "%s: tensor too large", fn);
  const size_t need = mxq::sqnr_workspace_bytes(rows * cols);
  if (need > mxq::sqnr_scratch_bytes())
    return fail(MXQ_ERR_INVALID_ARG, "%s: needs %zu bytes of workspace, above the library's %zu-byte scratch", fn,
                need, mxq::sqnr_scratch_bytes());
  if (!out3 || !aligned(out3, 8)) return fail(MXQ_ERR_INVALID_ARG, "%s: out3 must be a non-NULL 8-byte aligned pointer", fn);
  if (rows > 0 && cols > 0) {
    if (!ref || !test) return fail(MXQ_ERR_INVALID_ARG, "%s: ref/test is NULL", fn);
    if (!aligned(ref, 16) || !aligned(test, 16)) return fail(MXQ_ERR_INVALID_ARG, "%s: ref/test must be 16-byte aligned", fn);
  }
  void* ws = nullptr;
  hipError_t e = mxq::sqnr_scratch(&ws);
  if (e != hipSuccess) return hip_status(fn, e);
  return hip_status(fn, mxq::launch_sqnr(ref, test, rows, cols, ld_ref, ld_test, ws, out3, as_stream(stream)));
}

mxq_status mxq_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales, int64_t ld_scales,
                          int64_t rows, int64_t cols, uint16_t* y, int64_t ld_y, void* stream) {
  const char* fn = "mxq_dequantize";
  if (rows < 0 || cols < 0) return fail(MXQ_ERR_INVALID_ARG, "%s: negative size", fn);
  if (cols % 32 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: cols (%lld) must be a multiple of 32", fn, (long long)cols);
  if (ld_codes < cols / 2 || ld_scales < cols / 32 || ld_y < cols)
    return fail(MXQ_ERR_INVALID_ARG, "%s: pitch below the row width", fn);
  if (rows > kMaxDim || cols > kMaxDim || !pitch_ok(ld_codes) || !pitch_ok(ld_scales) || !pitch_ok(ld_y) ||
      rows * (cols / 32) >= ((int64_t)1 << 30))
    return fail(MXQ_ERR_INVALID_ARG, "%s: tensor too large", fn);
  if (rows > 0 && cols > 0) {
    if (!codes || !scales || !y) return fail(MXQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(codes, 4) || ld_codes % 4 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: codes must be 4-byte aligned", fn);
    if (!aligned(y, 16) || ld_y % 8 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: y base and pitch must be 16-byte aligned", fn);
  }
  return hip_status(fn, mxq::launch_dequantize(codes, ld_codes, scales, ld_scales, rows, cols, y, ld_y,
                                               as_stream(stream)));
}

mxq_status mxq_dequantize_fp8(const uint8_t* q, int64_t ld_q, float a_scale, int64_t rows, int64_t cols,
                              uint16_t* y, int64_t ld_y, void* stream) {
  const char* fn = "mxq_dequantize_fp8";
  if (rows < 0 || cols < 0) return fail(MXQ_ERR_INVALID_ARG, "%s: negative size", fn);
  if (cols % 16 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: cols (%lld) must be a multiple of 16", fn, (long long)cols);
  if (ld_q < cols || ld_y < cols) return fail(MXQ_ERR_INVALID_ARG, "%s: pitch below the row width", fn);
  if (!(a_scale == a_scale) || a_scale == __builtin_inff() || a_scale == -__builtin_inff())
    return fail(MXQ_ERR_INVALID_ARG, "%s: a_scale must be finite", fn);
  if (rows > kMaxDim || cols > kMaxDim || !pitch_ok(ld_q) || !pitch_ok(ld_y) || rows * (cols / 8) >= ((int64_t)1 << 32))
    return fail(MXQ_ERR_INVALID_ARG, "%s: tensor too large", fn);
  if (rows > 0 && cols > 0) {
    if (!q || !y) return fail(MXQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
    if (!aligned(q, 16) || ld_q % 16 != 0)
      return fail(MXQ_ERR_INVALID_ARG, "%s: q base and ld_q must be multiples of 16 bytes", fn);
    if (!aligned(y, 16) || ld_y % 8 != 0) return fail(MXQ_ERR_INVALID_ARG, "%s: y base and pitch must be 16-byte aligned", fn);
  }
  return hip_status(fn, mxq::launch_dequantize_fp8(q, ld_q, a_scale, rows, cols, y, ld_y, as_stream(stream)));
}

mxq_status mxq_mfma_ceiling(mxq_gemm_mode mode, const void* a, const uint8_t* a_scales, const void* w,
                            const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, int64_t waves, int64_t iters,
                            float* sink, void* stream) {
  const char* fn = "mxq_mfma_ceiling";
  if (mode != MXQ_GEMM_W4A4 && mode != MXQ_GEMM_W4A8 && mode != MXQ_GEMM_BF16)
    return fail(MXQ_ERR_UNSUPPORTED, "%s: unknown mode %d", fn, (int)mode);
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0)
    return fail(MXQ_ERR_INVALID_ARG, "%s: need M, N >= 1 and K a positive multiple of 32 (M=%lld N=%lld K=%lld)", fn,
                (long long)M, (long long)N, (long long)K);
  if (M > (int64_t)0x7FFFFFFF || N > (int64_t)0x7FFFFFFF || K > ((int64_t)1 << 21))
    return fail(MXQ_ERR_INVALID_ARG, "%s: dimension too large", fn);
  if (waves < 4 || waves % 4 != 0 || waves > ((int64_t)1 << 20))
    return fail(MXQ_ERR_INVALID_ARG, "%s: waves (%lld) must be a multiple of 4 in [4, 2^20]", fn, (long long)waves);
  if (iters < 1 || iters > ((int64_t)1 << 24))
    return fail(MXQ_ERR_INVALID_ARG, "%s: iters (%lld) must be in [1, 2^24]", fn, (long long)iters);
  mxq_status st;
  if ((st = check_operand(fn, "a", a, M, K, 16)) != MXQ_OK) return st;
  if ((st = check_operand(fn, "w", w, N, K, 16)) != MXQ_OK) return st;
  if (mode != MXQ_GEMM_BF16 && !w_scales) return fail(MXQ_ERR_INVALID_ARG, "%s: w_scales is NULL", fn);
  if (mode == MXQ_GEMM_W4A4 && !a_scales) return fail(MXQ_ERR_INVALID_ARG, "%s: a_scales is NULL", fn);
  if (!sink || !aligned(sink, 4)) return fail(MXQ_ERR_INVALID_ARG, "%s: sink must be a non-NULL 4-byte aligned pointer", fn);
  const mxq::GemmMode gm = mode == MXQ_GEMM_W4A4 ? mxq::GEMM_W4A4 : (mode == MXQ_GEMM_W4A8 ? mxq::GEMM_W4A8 : mxq::GEMM_BF16);
  return hip_status(fn, mxq::launch_mfma_ceiling(gm, a, a_scales, w, w_scales, M, N, K, waves, iters, sink,
                                                 as_stream(stream)));
}

}  // extern "C"
