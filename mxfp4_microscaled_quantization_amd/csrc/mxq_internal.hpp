// Internal launcher interface between the C ABI layer (mxq_api.hip) and the kernels.
// Launchers assume validated arguments, enqueue on `stream`, and return the HIP error
// of the launch (hipSuccess when nothing needed launching).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

hipError_t launch_quantize_mxfp4(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                 bool uos, hipStream_t stream);
hipError_t launch_quantize_mxfp4_rotated(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x, int n,
                                         uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                         bool uos, hipStream_t stream);
hipError_t launch_quantize_fp8(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x,
                               float inv_scale, uint8_t* q, int64_t ld_q, hipStream_t stream);
hipError_t launch_absmax(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x, float* out,
                         hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                             int64_t ld_scales, int64_t rows, int64_t cols, uint16_t* y, int64_t ld_y,
                             hipStream_t stream);
hipError_t launch_dequantize_fp8(const uint8_t* q, int64_t ld_q, float a_scale, int64_t rows, int64_t cols,
                                 uint16_t* y, int64_t ld_y, hipStream_t stream);

enum GemmMode { GEMM_W4A4 = 0, GEMM_W4A8 = 1, GEMM_BF16 = 2 };
hipError_t launch_gemm(GemmMode mode, const void* a, const uint8_t* a_scales, const void* w,
                       const uint8_t* w_scales, float a_scale, int64_t M, int64_t N, int64_t K,
                       uint16_t* out, int64_t ld_out, hipStream_t stream);

// W4A4 with the activation quantization fused in: `a` is rows x K of bf16 (or binary32),
// pitch ld_a elements; uos selects the UOS scale rule.
hipError_t launch_gemm_w4a4_fused(const void* a, bool f32, int64_t ld_a, const uint8_t* w, const uint8_t* w_scales,
                                  int64_t M, int64_t N, int64_t K, bool uos, uint16_t* out, int64_t ld_out,
                                  hipStream_t stream);

// Register-only MFMA loop on fragments gathered from a GEMM call's operand planes
// (waves a multiple of 4; sink: one float per lane).
hipError_t launch_mfma_ceiling(GemmMode mode, const void* a, const uint8_t* a_scales, const void* w,
                               const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, int64_t waves, int64_t iters,
                               float* sink, hipStream_t stream);

size_t sqnr_workspace_bytes(int64_t n);
// The library's own SQNR workspace on the current device (a static device array,
// sqnr_scratch_bytes() long): its device address, looked up once per device.
size_t sqnr_scratch_bytes();
hipError_t sqnr_scratch(void** ptr);
hipError_t launch_sqnr(const uint16_t* ref, const uint16_t* test, int64_t rows, int64_t cols,
                       int64_t ld_ref, int64_t ld_test, void* ws, double* out3, hipStream_t stream);

}  // namespace mxq
