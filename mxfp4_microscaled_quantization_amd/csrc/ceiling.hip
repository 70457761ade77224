// MFMA throughput ceiling on the operand bits of a GEMM call (a measurement aid, not part
// of the quantize / GEMM path).
//
// Under these GEMMs the MI355X runs below its top clock: it holds its power, and the
// energy of an MFMA grows with the number of operand bits that toggle.  The dense peak is
// therefore out of reach with real operands even without memory traffic.  This kernel
// measures what the matrix cores sustain on the bits of a given call: every lane gathers
// the bytes one lane of the GEMM's MFMA holds -- 4 weight and 4 activation fragments
// from pseudo-random rows and 32-element blocks of the operand planes, with their scale
// bytes -- and runs the GEMM's instruction on them in registers (32 x 32 x 64 scaled MFMAs
// for W4A4 / W4A8, 16 x 16 x 32 for bf16), cycling through the 4 x 4 fragment pairs as
// a wave tile does.  The fragments stay fixed across
// iterations, so operands toggle a little less than in the GEMM: the ceiling is, if
// anything, optimistic.
#include <type_traits>

#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {
namespace {

struct CeilingParams {
  const uint8_t *a, *a_scales, *w, *w_scales;
  int64_t M, N, K;
  int iters;
  float* sink;
};

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// The BYTES-byte chunk c of row r of a plane of rows x row_bytes bytes, for a row and a
// chunk drawn from h.  FP4 and FP8 chunks (16 / 32 bytes) are one 32-element block each,
// so c is also the index of the chunk's scale byte in its row.
template <int BYTES>
__device__ __forceinline__ v8i gather(const uint8_t* base, int64_t rows, int64_t row_bytes, uint32_t h, int64_t& r,
                                      int64_t& c) {
  r = (int64_t)(h % (uint32_t)rows);
  c = (int64_t)(mix32(h) % (uint32_t)(row_bytes / BYTES));
  const v4i* q = reinterpret_cast<const v4i*>(base + r * row_bytes + c * BYTES);
  const v4i lo = q[0];
  v8i v = {lo[0], lo[1], lo[2], lo[3], 0, 0, 0, 0};
  if constexpr (BYTES == 32) {
    const v4i hi = q[1];
    v[4] = hi[0];
    v[5] = hi[1];
    v[6] = hi[2];
    v[7] = hi[3];
  }
  return v;
}

// One wave per SIMD for the scaled modes (256 accumulator registers, as in their GEMM);
// two for bf16, as in its GEMM, which keeps the accumulators in VGPRs
template <int MODE>
__global__ __launch_bounds__(256, MODE == GEMM_BF16 ? 2 : 1) void mfma_ceiling_kernel(CeilingParams p) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  // bytes per lane fragment and per row of each operand plane
  constexpr int WB = 16;                                        // fp4: 32 elements; bf16: 8
  constexpr int AB = MODE == GEMM_W4A8 ? 32 : 16;               // fp8: 32 elements
  const int64_t w_rb = MODE == GEMM_BF16 ? 2 * p.K : p.K / 2;
  const int64_t a_rb = MODE == GEMM_BF16 ? 2 * p.K : (MODE == GEMM_W4A8 ? p.K : p.K / 2);
  const int64_t sc_rb = p.K / 32;
  v8i fw[4], fa[4];
  int scw[4], sca[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int64_t r, c;
    fw[i] = gather<WB>(p.w, p.N, w_rb, mix32(gid * 16u + (uint32_t)i), r, c);
    scw[i] = MODE == GEMM_BF16 ? 127 : (int)p.w_scales[r * sc_rb + c];
    fa[i] = gather<AB>(p.a, p.M, a_rb, mix32(gid * 16u + 8u + (uint32_t)i), r, c);
    sca[i] = MODE == GEMM_W4A4 ? (int)p.a_scales[r * sc_rb + c] : 127;
  }
  // the scaled modes' GEMM runs 32 x 32 x 64 MFMAs, the bf16 reference 16 x 16 x 32
  using Acc = typename std::conditional<MODE == GEMM_BF16, v4f, v16f>::type;
  constexpr int AE = MODE == GEMM_BF16 ? 4 : 16;
  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < AE; ++e) acc[i][j][e] = 0.0f;
  for (int it = 0; it < p.iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (MODE == GEMM_W4A4)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[i], fa[j], acc[i][j], 4, 4, 0, scw[i], 0,
                                                                      sca[j]);
        else if constexpr (MODE == GEMM_W4A8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[i], fa[j], acc[i][j], 4, 0, 0, scw[i], 0, 127);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(fw[i], fw[i], 0, 1, 2, 3)),
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(fa[j], fa[j], 0, 1, 2, 3)), acc[i][j], 0, 0, 0);
      }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < AE; ++e) s += acc[i][j][e];
  p.sink[gid] = s;
}

}  // namespace

hipError_t launch_mfma_ceiling(GemmMode mode, const void* a, const uint8_t* a_scales, const void* w,
                               const uint8_t* w_scales, int64_t M, int64_t N, int64_t K, int64_t waves, int64_t iters,
                               float* sink, hipStream_t stream) {
  CeilingParams p{static_cast<const uint8_t*>(a), a_scales, static_cast<const uint8_t*>(w), w_scales, M, N, K,
                  (int)iters, sink};
  const dim3 grid((unsigned)(waves / 4)), block(256);
  switch (mode) {
    case GEMM_W4A4:
      hipLaunchKernelGGL(mfma_ceiling_kernel<GEMM_W4A4>, grid, block, 0, stream, p);
      break;
    case GEMM_W4A8:
      hipLaunchKernelGGL(mfma_ceiling_kernel<GEMM_W4A8>, grid, block, 0, stream, p);
      break;
    case GEMM_BF16:
      hipLaunchKernelGGL(mfma_ceiling_kernel<GEMM_BF16>, grid, block, 0, stream, p);
      break;
  }
  return hipGetLastError();
}

}  // namespace mxq
