// Bandwidth-bound element kernels for gfx950: MXFP4 block quantization, static FP8 E4M3
// quantization, absolute maximum (static-scale calibration) and MXFP4 dequantization.
//
// MXFP4 rule ("AMD Quark: 1.92x faster FLUX.1-dev with MXFP4 on Instinct MI350", section
// "What is MXFP4": 32-element blocks share one scale; "MXAttention ...", section "What it
// actually does": the scale is an E8M0 power of two): per block, the scale byte is
// s = max(E(amax) - 2, 0) with E the biased exponent field of amax, i.e.
// X = 2^(floor(log2 amax) - 2) clamped at 2^-127, and every element becomes the E2M1
// value nearest to x / X (ties to even, saturating at +-6).
//
// UOS variant ("MXAttention ...", section "What it actually does": a data-free scaling
// boundary Qmax = 7.25): X is the smallest power of two with amax <= 7.25 X.  With
// amax = m 2^e, m in [1, 2), that is 2^(e-2) when 4m <= 7.25 and 2^(e-1) otherwise, so
// the byte is the OCP byte plus one exactly when the significand of amax exceeds 1.8125
// (fraction field above 0x680000 in binary32, 0x68 in bf16), floored at 0 as before.
//
// Mapping: four consecutive lanes own one 32-element block (8 elements, 16 bytes of
// bf16, per lane), so each wave load instruction moves 1 KB of contiguous input and the
// block maximum is a 2-step DPP reduction inside the quad.  The E2M1 rounding is the
// gfx950 conversion v_cvt_scalef32_pk_fp4_f32, which computes round-to-nearest-even of
// x / scale with saturation for power-of-two scales (including the subnormal 2^-127), two
// elements per instruction (bf16 inputs are widened exactly first).
#include <type_traits>

#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {
namespace {

constexpr int kThreads = 256;         // absmax_kernel
// mx_quantize_kernel: 512-thread workgroups, 8 blocks in flight per quad (77 % of HBM
// against 63 % with 256 threads and 4 blocks); the FP8 kernel runs 1024-thread workgroups.
constexpr int kMxThreads = 512;
constexpr int kMxUnroll = 8;
constexpr int kMxBlocksPerIter = kMxThreads / 4 * kMxUnroll;
constexpr int kFp8Threads = 1024;
constexpr int kFp8Unroll = 2;     // chunks of 16 per lane per pass (72 % of HBM against 69 % for one)
// dequantize_kernel: 8 quarter-blocks per lane per pass in 512-thread workgroups (71 % of
// HBM against 58 % for one quarter per lane and 256 threads)
constexpr int kDqThreads = 512;
constexpr int kDqUnroll = 8;
// mx_quantize_rot_kernel: 512-thread workgroups, 4 blocks in flight per quad, every load
// of an iteration issued before its butterflies (66 % of HBM for n = 64 against 61 % with
// 256 threads and each block's load, butterfly and store in turn)
constexpr int kRotThreads = 512;
constexpr int kRotUnroll = 4;

__device__ __forceinline__ float lo_f32(int pair) { return __uint_as_float((unsigned)pair << 16); }
__device__ __forceinline__ float hi_f32(int pair) { return __uint_as_float((unsigned)pair & 0xFFFF0000u); }

// ---------------------------------------------------------------------------------
// MXFP4 quantization.  F32 selects binary32 input (else bf16); UOS the 7.25 boundary.
template <bool F32, bool UOS>
__global__ __launch_bounds__(kMxThreads) void mx_quantize_kernel(
    const void* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, uint32_t blocks_per_row, int64_t total_blocks,
    int contiguous) {
  const int tid = threadIdx.x;
  const int q = tid & 3;                       // quarter of the block owned by this lane
  const int64_t stride = (int64_t)gridDim.x * kMxBlocksPerIter;
  for (int64_t base = (int64_t)blockIdx.x * kMxBlocksPerIter; base < total_blocks; base += stride) {
    int64_t xo[kMxUnroll], co[kMxUnroll], so[kMxUnroll];
    bool ok[kMxUnroll];
    v4i d0[kMxUnroll], d1[kMxUnroll];
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      const int64_t b = base + u * (kMxThreads / 4) + (tid >> 2);
      ok[u] = b < total_blocks;
      if (contiguous) {
        xo[u] = b * 32 + q * 8;
        co[u] = b * 16 + q * 4;
        so[u] = b;
      } else {
        const uint32_t bb = (uint32_t)b;
        const uint32_t row = bb / blocks_per_row;
        const uint32_t blk = bb - row * blocks_per_row;
        xo[u] = (int64_t)row * ld_x + blk * 32 + q * 8;
        co[u] = (int64_t)row * ld_codes + blk * 16 + q * 4;
        so[u] = (int64_t)row * ld_scales + blk;
      }
      d0[u] = v4i{0, 0, 0, 0};
      d1[u] = v4i{0, 0, 0, 0};
      if (ok[u]) {
        if (F32) {
          const v4i* p = reinterpret_cast<const v4i*>(static_cast<const float*>(x) + xo[u]);
          d0[u] = __builtin_nontemporal_load(p);
          d1[u] = __builtin_nontemporal_load(p + 1);
        } else {
          d0[u] = __builtin_nontemporal_load(
              reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(x) + xo[u]));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kMxUnroll; ++u) {
      unsigned amax, e, bump;
      if (F32) {
        unsigned m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          m = max(m, (unsigned)d0[u][i] & 0x7FFFFFFFu);
          m = max(m, (unsigned)d1[u][i] & 0x7FFFFFFFu);
        }
        amax = quad_max_u32(m);
        e = amax >> 23;
        bump = (amax & 0x7FFFFFu) > 0x680000u ? 1u : 0u;
      } else {
        v2h m = {0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m = __builtin_elementwise_max(m, __builtin_bit_cast(v2h, (unsigned)d0[u][i] & 0x7FFF7FFFu));
        amax = quad_max_u32(max((unsigned)m[0], (unsigned)m[1]));
        e = amax >> 7;
        bump = (amax & 0x7Fu) > 0x68u ? 1u : 0u;
      }
      const unsigned s = UOS ? scale_byte_uos(e, bump) : scale_byte_from_exp(e);
      const float scale = e8m0_to_f32(s);
      unsigned r = 0;
      if (F32) {
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __int_as_float(d0[u][0]), __int_as_float(d0[u][1]), scale, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __int_as_float(d0[u][2]), __int_as_float(d0[u][3]), scale, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __int_as_float(d1[u][0]), __int_as_float(d1[u][1]), scale, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __int_as_float(d1[u][2]), __int_as_float(d1[u][3]), scale, 3);
      } else {
        // bf16 pairs are widened exactly to binary32 (a shift / a mask) and converted
        // with the f32 form, whose destination-byte select places byte k of the word
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo_f32(d0[u][0]), hi_f32(d0[u][0]), scale, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo_f32(d0[u][1]), hi_f32(d0[u][1]), scale, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo_f32(d0[u][2]), hi_f32(d0[u][2]), scale, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, lo_f32(d0[u][3]), hi_f32(d0[u][3]), scale, 3);
      }
      if (ok[u]) {
        // codes are not read again by this kernel: stream them past the caches
        __builtin_nontemporal_store(r, reinterpret_cast<unsigned*>(codes + co[u]));
        if (q == 0) scales[so[u]] = (uint8_t)s;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Fixed block-Hadamard rotation, then MXFP4 ("AMD Quark adds native W4A8 mixed-precision
// for Wan2.2 ...", section "Quark quantization pipeline and mixed-precision selection":
// a fixed Hadamard rotation as the transform condition; "Exp 2026-08-22 W4A4 Reference
// Model", section "Status": block-Hadamard with per-group scales).  Every run of N
// consecutive elements along K becomes x H_N / sqrt(N) (Sylvester H_N, N = 16, 64, 256,
// so 1/sqrt(N) is a power of two), formed in binary32 by the radix-2 butterfly in stage
// order h = 1, 2, 4, ...: the pair (i, i + h) becomes (x_i + x_{i+h}, x_i - x_{i+h}).
// The rotated values are then quantized as binary32 input.  Same lane mapping as
// mx_quantize_kernel (4 lanes per 32-element block, 8 elements per lane): stages h < 8
// stay in the lane, stages h >= 8 pair lane l with lane l ^ (h / 8).  A run never straddles
// a row (K % N == 0) and starts at a multiple of N / 8 lanes.  Adds and the final scaling
// are explicitly rounded (no contraction into fused operations).
// value of lane l ^ D (D < 32): DPP inside a row of 16 lanes (quad permutes for 1 and 2,
// row shifts for 4, a row rotation for 8), a permute through the LDS crossbar beyond
template <int D>
__device__ __forceinline__ float lane_xor(float v, int lane) {
  const int b = __float_as_int(v);
  if constexpr (D == 1) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));    // quad_perm [1,0,3,2]
  } else if constexpr (D == 2) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));    // quad_perm [2,3,0,1]
  } else if constexpr (D == 4) {
    const int up = __builtin_amdgcn_mov_dpp(b, 0x104, 0xF, 0xF, true);          // row_shl:4 (lane + 4)
    const int dn = __builtin_amdgcn_mov_dpp(b, 0x114, 0xF, 0xF, true);          // row_shr:4 (lane - 4)
    return __int_as_float((lane & 4) ? dn : up);
  } else if constexpr (D == 8) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true));   // row_ror:8
  } else {
    // through the LDS crossbar (ds_bpermute): measured faster here than the gfx950
    // v_permlane16_swap, whose operand copies and hazard waits serialize the exchanges
    return __shfl_xor(v, D);
  }
}

template <bool F32, int N, bool UOS, int THREADS, int UNROLL>
__global__ __launch_bounds__(THREADS) void mx_quantize_rot_kernel(
    const void* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, uint32_t blocks_per_row, int64_t total_blocks,
    int contiguous) {
  static_assert(N == 16 || N == 64 || N == 256, "rotation runs of 16, 64 or 256");
  constexpr float kNorm = N == 16 ? 0.25f : (N == 64 ? 0.125f : 0.0625f);   // 1 / sqrt(N)
  constexpr int BLOCKS_PER_ITER = THREADS / 4 * UNROLL;
  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int lane = tid & 63;
  const int64_t stride = (int64_t)gridDim.x * BLOCKS_PER_ITER;
  for (int64_t base = (int64_t)blockIdx.x * BLOCKS_PER_ITER; base < total_blocks; base += stride) {
    // every block's loads first, then the butterflies and stores
    int64_t co[UNROLL], so[UNROLL];
    bool ok[UNROLL];
    v4i d0[UNROLL], d1[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t b = base + u * (THREADS / 4) + (tid >> 2);
      ok[u] = b < total_blocks;
      int64_t xo;
      if (contiguous) {
        xo = b * 32 + q * 8;
        co[u] = b * 16 + q * 4;
        so[u] = b;
      } else {
        const uint32_t bb = (uint32_t)b;
        const uint32_t row = bb / blocks_per_row;
        const uint32_t blk = bb - row * blocks_per_row;
        xo = (int64_t)row * ld_x + blk * 32 + q * 8;
        co[u] = (int64_t)row * ld_codes + blk * 16 + q * 4;
        so[u] = (int64_t)row * ld_scales + blk;
      }
      d0[u] = v4i{0, 0, 0, 0};
      d1[u] = v4i{0, 0, 0, 0};
      if (ok[u]) {
        if (F32) {
          const v4i* p = reinterpret_cast<const v4i*>(static_cast<const float*>(x) + xo);
          d0[u] = __builtin_nontemporal_load(p);
          d1[u] = __builtin_nontemporal_load(p + 1);
        } else {
          d0[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(x) + xo));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      float v[8];
      if (F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = __int_as_float(d0[u][i]);
          v[4 + i] = __int_as_float(d1[u][i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[2 * i] = lo_f32(d0[u][i]);
          v[2 * i + 1] = hi_f32(d0[u][i]);
        }
      }
      // stages h = 1, 2, 4 inside the lane
#pragma unroll
      for (int h = 1; h < 8; h *= 2)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((i & h) == 0) {
            const float a = v[i], c = v[i + h];
            v[i] = __fadd_rn(a, c);
            v[i + h] = __fsub_rn(a, c);
          }
      // stages h = 8, 16, ... across lanes l and l ^ (h / 8); the lower index keeps the sum
      auto cross = [&](auto d_tag) {
        constexpr int D = decltype(d_tag)::value;
        if constexpr (D < N / 8) {
          const bool upper = (lane & D) != 0;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float other = lane_xor<D>(v[i], lane);
            v[i] = upper ? __fsub_rn(other, v[i]) : __fadd_rn(v[i], other);
          }
        }
      };
      cross(std::integral_constant<int, 1>{});
      cross(std::integral_constant<int, 2>{});
      cross(std::integral_constant<int, 4>{});
      cross(std::integral_constant<int, 8>{});
      cross(std::integral_constant<int, 16>{});
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __fmul_rn(v[i], kNorm);
      // MXFP4 of the rotated binary32 values (as mx_quantize_kernel)
      unsigned m = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(v[i]) & 0x7FFFFFFFu);
      const unsigned amax = quad_max_u32(m);
      const unsigned e = amax >> 23;
      const unsigned s = UOS ? scale_byte_uos(e, (amax & 0x7FFFFFu) > 0x680000u ? 1u : 0u) : scale_byte_from_exp(e);
      const float scale = e8m0_to_f32(s);
      unsigned r = 0;
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[0], v[1], scale, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], scale, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], scale, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], scale, 3);
      if (ok[u]) {
        __builtin_nontemporal_store(r, reinterpret_cast<unsigned*>(codes + co[u]));
        if (q == 0) scales[so[u]] = (uint8_t)s;
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Static FP8 E4M3: q = E4M3_RNE(clamp(fl32(x * inv_scale), -448, 448)).  The clamp makes
// the gfx950 conversion saturate (it returns NaN past the rounding edge otherwise); the
// clamp keeps the sign of zero.  16 elements per lane, one 16-byte store.
template <bool F32>
__global__ __launch_bounds__(kFp8Threads) void fp8_quantize_kernel(
    const void* __restrict__ x, int64_t ld_x, float inv_scale, uint8_t* __restrict__ out, int64_t ld_q,
    uint32_t chunks_per_row, int64_t total_chunks, int contiguous) {
  // each lane takes kFp8Unroll chunks of 16 elements per pass, loads first
  const int64_t stride = (int64_t)gridDim.x * kFp8Threads * kFp8Unroll;
  for (int64_t c0 = (int64_t)blockIdx.x * kFp8Threads * kFp8Unroll + threadIdx.x; c0 < total_chunks; c0 += stride) {
    v4i d[kFp8Unroll][4];
    int64_t qo[kFp8Unroll];
    bool ok[kFp8Unroll];
#pragma unroll
    for (int u = 0; u < kFp8Unroll; ++u) {
      const int64_t c = c0 + (int64_t)u * kFp8Threads;
      ok[u] = c < total_chunks;
      int64_t xo;
      if (contiguous) {
        xo = c * 16;
        qo[u] = c * 16;
      } else {
        const uint32_t cc = (uint32_t)c;
        const uint32_t row = cc / chunks_per_row;
        const uint32_t col = cc - row * chunks_per_row;
        xo = (int64_t)row * ld_x + col * 16;
        qo[u] = (int64_t)row * ld_q + col * 16;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) d[u][i] = v4i{0, 0, 0, 0};
      if (ok[u]) {
        if (F32) {
          const v4i* p = reinterpret_cast<const v4i*>(static_cast<const float*>(x) + xo);
#pragma unroll
          for (int i = 0; i < 4; ++i) d[u][i] = __builtin_nontemporal_load(p + i);
        } else {
          const v4i* p = reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(x) + xo);
          d[u][0] = __builtin_nontemporal_load(p);
          d[u][1] = __builtin_nontemporal_load(p + 1);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kFp8Unroll; ++u) {
      float v[16];
      if (F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v[4 * i + jj] = __int_as_float(d[u][i][jj]);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            v[8 * i + 2 * jj] = __uint_as_float((unsigned)d[u][i][jj] << 16);
            v[8 * i + 2 * jj + 1] = __uint_as_float((unsigned)d[u][i][jj] & 0xFFFF0000u);
          }
      }
      v4i o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float y[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) y[jj] = __builtin_amdgcn_fmed3f(v[4 * i + jj] * inv_scale, -448.0f, 448.0f);
        int r = 0;
        r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], r, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);
        o[i] = r;
      }
      if (ok[u]) __builtin_nontemporal_store(o, reinterpret_cast<v4i*>(out + qo[u]));
    }
  }
}

// ---------------------------------------------------------------------------------
// max |x| over a tensor (8 elements per lane per step); the result is combined with an
// integer atomic max on the binary32 bit pattern, which orders non-negative floats.
__global__ void absmax_init_kernel(float* out) { *out = 0.0f; }

template <bool F32>
__global__ __launch_bounds__(kThreads) void absmax_kernel(const void* __restrict__ x, int64_t ld_x,
                                                          uint32_t chunks_per_row, int64_t total_chunks,
                                                          int contiguous, unsigned* __restrict__ out) {
  __shared__ unsigned red[kThreads / 64];
  unsigned m = 0;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < total_chunks; c += stride) {
    int64_t xo;
    if (contiguous) {
      xo = c * 8;
    } else {
      const uint32_t cc = (uint32_t)c;
      const uint32_t row = cc / chunks_per_row;
      xo = (int64_t)row * ld_x + (int64_t)(cc - row * chunks_per_row) * 8;
    }
    if (F32) {
      const v4i* p = reinterpret_cast<const v4i*>(static_cast<const float*>(x) + xo);
      const v4i a = p[0], b = p[1];
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, max((unsigned)a[i] & 0x7FFFFFFFu, (unsigned)b[i] & 0x7FFFFFFFu));
    } else {
      const v4i a = *reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(x) + xo);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        m = max(m, max(((unsigned)a[i] & 0x7FFFu) << 16, (unsigned)a[i] & 0x7FFF0000u));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned r = red[0];
    for (int i = 1; i < kThreads / 64; ++i) r = max(r, red[i]);
    atomicMax(out, r);
  }
}

// ---------------------------------------------------------------------------------
// MXFP4 -> bf16: e2m1(code) * 2^(s - 127).  The product is formed in binary32 (exact:
// at most 3 significant bits, exponent within binary32's range down to the subnormal
// 2^-128) and narrowed to bf16 with round to nearest even (exact in range).
__global__ __launch_bounds__(kDqThreads) void dequantize_kernel(
    const uint8_t* __restrict__ codes, int64_t ld_codes, const uint8_t* __restrict__ scales,
    int64_t ld_scales, uint16_t* __restrict__ y, int64_t ld_y, uint32_t blocks_per_row,
    int64_t total_quarters) {
  // each lane takes kDqUnroll quarters (8 elements each) per pass, loads first
  const int64_t stride = (int64_t)gridDim.x * kDqThreads * kDqUnroll;
  for (int64_t g0 = (int64_t)blockIdx.x * kDqThreads * kDqUnroll + threadIdx.x; g0 < total_quarters; g0 += stride) {
    unsigned c[kDqUnroll], s[kDqUnroll];
    int64_t yo[kDqUnroll];
    bool ok[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const int64_t g = g0 + (int64_t)u * kDqThreads;
      ok[u] = g < total_quarters;
      const int64_t b = g >> 2;
      const int q = (int)(g & 3);
      const uint32_t row = (uint32_t)(b / blocks_per_row);
      const uint32_t blk = (uint32_t)(b - (int64_t)row * blocks_per_row);
      c[u] = ok[u] ? *reinterpret_cast<const unsigned*>(codes + (int64_t)row * ld_codes + blk * 16 + q * 4) : 0u;
      s[u] = ok[u] ? scales[(int64_t)row * ld_scales + blk] : 0u;
      yo[u] = (int64_t)row * ld_y + blk * 32 + q * 8;
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      // 2 * |e2m1| for magnitude codes 0..7 is 0,1,2,3,4,6,8,12: one nibble each
      const unsigned sv = s[u];
      const float half_scale = sv >= 2 ? __uint_as_float((sv - 1) << 23) : (sv == 1 ? 0x1p-127f : 0x1p-128f);
      const float sc = sv == 255 ? __uint_as_float(0x7FC00000u) : half_scale;
      v4i o;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float f[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const unsigned code = (c[u] >> (8 * i + 4 * h)) & 0xF;
          const float mag = (float)((0xC8643210u >> (4 * (code & 7))) & 0xF) * sc;
          f[h] = (code & 8) ? -mag : mag;
        }
        o[i] = (int)pack_bf16x2(f[0], f[1]);
      }
      // the output is not read again here: stream it past the caches
      if (ok[u]) __builtin_nontemporal_store(o, reinterpret_cast<v4i*>(y + yo[u]));
    }
  }
}

int grid_for(int64_t work_items, int64_t per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  const int64_t cap = 256 * 64;  // enough resident waves to cover HBM latency
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t launch_quantize_mxfp4(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                 bool uos, hipStream_t stream) {
  const int64_t bpr = cols / 32;
  const int64_t total = rows * bpr;
  if (total == 0) return hipSuccess;
  const int contiguous = (ld_x == cols && ld_codes == cols / 2 && ld_scales == bpr) ? 1 : 0;
  const int grid = grid_for(total, kMxBlocksPerIter);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kMxThreads), 0, stream, x, ld_x, codes, ld_codes, scales, ld_scales,
                       (uint32_t)bpr, total, contiguous);
  };
  if (f32)
    uos ? go(mx_quantize_kernel<true, true>) : go(mx_quantize_kernel<true, false>);
  else
    uos ? go(mx_quantize_kernel<false, true>) : go(mx_quantize_kernel<false, false>);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4_rotated(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x, int n,
                                         uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                         bool uos, hipStream_t stream) {
  const int64_t bpr = cols / 32;
  const int64_t total = rows * bpr;
  if (total == 0) return hipSuccess;
  const int contiguous = (ld_x == cols && ld_codes == cols / 2 && ld_scales == bpr) ? 1 : 0;
  constexpr int T = kRotThreads, U = kRotUnroll;
  const int grid = grid_for(total, T / 4 * U);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(T), 0, stream, x, ld_x, codes, ld_codes, scales, ld_scales,
                       (uint32_t)bpr, total, contiguous);
  };
  auto pick_rule = [&](auto f32_tag, auto n_tag) {
    constexpr bool F = decltype(f32_tag)::value;
    constexpr int NN = decltype(n_tag)::value;
    uos ? go(mx_quantize_rot_kernel<F, NN, true, T, U>) : go(mx_quantize_rot_kernel<F, NN, false, T, U>);
  };
  auto pick_n = [&](auto f32_tag) {
    if (n == 16)
      pick_rule(f32_tag, std::integral_constant<int, 16>{});
    else if (n == 64)
      pick_rule(f32_tag, std::integral_constant<int, 64>{});
    else
      pick_rule(f32_tag, std::integral_constant<int, 256>{});
  };
  if (f32)
    pick_n(std::true_type{});
  else
    pick_n(std::false_type{});
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x,
                               float inv_scale, uint8_t* q, int64_t ld_q, hipStream_t stream) {
  const int64_t cpr = cols / 16;
  const int64_t total = rows * cpr;
  if (total == 0) return hipSuccess;
  const int contiguous = (ld_x == cols && ld_q == cols) ? 1 : 0;
  const int grid = grid_for(total, kFp8Threads * kFp8Unroll);
  if (f32)
    hipLaunchKernelGGL(fp8_quantize_kernel<true>, dim3(grid), dim3(kFp8Threads), 0, stream, x, ld_x, inv_scale,
                       q, ld_q, (uint32_t)cpr, total, contiguous);
  else
    hipLaunchKernelGGL(fp8_quantize_kernel<false>, dim3(grid), dim3(kFp8Threads), 0, stream, x, ld_x, inv_scale,
                       q, ld_q, (uint32_t)cpr, total, contiguous);
  return hipGetLastError();
}

hipError_t launch_absmax(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x, float* out,
                         hipStream_t stream) {
  hipLaunchKernelGGL(absmax_init_kernel, dim3(1), dim3(1), 0, stream, out);
  const int64_t cpr = cols / 8;
  const int64_t total = rows * cpr;
  if (total > 0) {
    const int contiguous = ld_x == cols ? 1 : 0;
    const int grid = grid_for(total, kThreads * 4);
    if (f32)
      hipLaunchKernelGGL(absmax_kernel<true>, dim3(grid), dim3(kThreads), 0, stream, x, ld_x, (uint32_t)cpr,
                         total, contiguous, reinterpret_cast<unsigned*>(out));
    else
      hipLaunchKernelGGL(absmax_kernel<false>, dim3(grid), dim3(kThreads), 0, stream, x, ld_x, (uint32_t)cpr,
                         total, contiguous, reinterpret_cast<unsigned*>(out));
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, int64_t ld_codes, const uint8_t* scales,
                             int64_t ld_scales, int64_t rows, int64_t cols, uint16_t* y, int64_t ld_y,
                             hipStream_t stream) {
  const int64_t bpr = cols / 32;
  const int64_t total = rows * bpr * 4;
  if (total == 0) return hipSuccess;
  const int grid = grid_for(total, kDqThreads * kDqUnroll);
  hipLaunchKernelGGL(dequantize_kernel, dim3(grid), dim3(kDqThreads), 0, stream, codes, ld_codes, scales,
                     ld_scales, y, ld_y, (uint32_t)bpr, total);
  return hipGetLastError();
}

}  // namespace mxq
