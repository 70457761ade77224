// Bandwidth-bound element kernels for gfx950: MXFP4 block quantization, static FP8 E4M3
// quantization, absolute maximum (static-scale calibration), and MXFP4 and FP8 E4M3
// dequantization (the quantize-dequantize emulation steps).
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
// mx_quantize_kernel: 1024-thread workgroups, 4 blocks in flight per quad, buffer loads
// for packed rows (80 % of HBM; 512 threads with 8 blocks 77 %, 256 threads with 8 or 16
// blocks 72-74 %)
constexpr int kMxThreads = 1024;
constexpr int kMxUnroll = 4;
constexpr int kMxBlocksPerIter = kMxThreads / 4 * kMxUnroll;
// fp8_quantize_kernel: units of 8 elements (one 16-byte bf16 load and one 8-byte store per
// lane, both contiguous across the wave), 4 units per lane per pass in 512-thread
// workgroups: 75-78 % of HBM against 72-74 % for 16-element units (two 16-byte loads per
// lane, each instruction covering half of every line it touches)
constexpr int kFp8Threads = 512;
constexpr int kFp8Unroll = 4;
// dequantize_kernel: 4 quarter-blocks per lane per pass in 1024-thread workgroups, loads
// first (72 % of HBM; 512 threads with 2, 8 or 16 quarters and 256 threads with 8 within
// 4 % of it; 58 % for one quarter per lane and 256 threads)
constexpr int kDqThreads = 1024;
constexpr int kDqUnroll = 4;
// dequantize_fp8_kernel: 8 codes (8 bytes in, 16 bytes out) per lane per unit, 4 units
// per lane per pass, loads first, 1024-thread workgroups (the same sweep: within 4 %)
constexpr int kDq8Threads = 1024;
constexpr int kDq8Unroll = 4;

// ---------------------------------------------------------------------------------
// MXFP4 quantization.  F32 selects binary32 input (else bf16); UOS the 7.25 boundary;
// CONTIG packed rows (linear offsets, buffer loads), else one 32-bit division per block.
template <bool F32, bool UOS, bool CONTIG>
__global__ __launch_bounds__(kMxThreads) void mx_quantize_kernel(
    const void* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, uint32_t blocks_per_row, int64_t total_blocks) {
  constexpr int T = kMxThreads, U = kMxUnroll, BPI = kMxBlocksPerIter;
  const int tid = threadIdx.x;
  const int q = tid & 3;
  const int64_t stride = (int64_t)gridDim.x * BPI;
  for (int64_t base = (int64_t)blockIdx.x * BPI; base < total_blocks; base += stride) {
    v4i d0[U], d1[U];
    int64_t co[U], so[U];
    bool ok[U];
    // packed rows: the pass's BPI blocks are one span, read through a buffer descriptor
    // whose range check zero-fills past the last block (no per-load branch)
    const int64_t left = total_blocks - base;
    const uint32_t nb = left <= 0 ? 0u : (uint32_t)(left < BPI ? left : BPI);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(x) + base * (F32 ? 128 : 64), nb * (F32 ? 128u : 64u));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int lb = u * (T / 4) + (tid >> 2);          // block within the pass
      const int64_t b = base + lb;
      ok[u] = b < total_blocks;
      if (CONTIG) {
        co[u] = b * 16 + q * 4;
        so[u] = b;
        if (F32) {
          d0[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, lb * 128 + q * 32, 0, 2));
          d1[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, lb * 128 + q * 32 + 16, 0, 2));
        } else {
          d0[u] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, lb * 64 + q * 16, 0, 2));
          d1[u] = v4i{0, 0, 0, 0};
        }
      } else {
        const uint32_t bb = (uint32_t)b;
        const uint32_t row = bb / blocks_per_row;
        const uint32_t blk = bb - row * blocks_per_row;
        const int64_t xo = (int64_t)row * ld_x + blk * 32 + q * 8;
        co[u] = (int64_t)row * ld_codes + blk * 16 + q * 4;
        so[u] = (int64_t)row * ld_scales + blk;
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
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
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
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo_f32(d0[u][0]), bf16_hi_f32(d0[u][0]), scale, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo_f32(d0[u][1]), bf16_hi_f32(d0[u][1]), scale, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo_f32(d0[u][2]), bf16_hi_f32(d0[u][2]), scale, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo_f32(d0[u][3]), bf16_hi_f32(d0[u][3]), scale, 3);
      }
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
// clamp keeps the sign of zero.  8 elements per lane and unit: one 16-byte bf16 load, one
// 8-byte store.
template <bool F32>
__global__ __launch_bounds__(kFp8Threads) void fp8_quantize_kernel(
    const void* __restrict__ x, int64_t ld_x, float inv_scale, uint8_t* __restrict__ out, int64_t ld_q,
    uint32_t units_per_row, int64_t total_units, int contiguous) {
  constexpr int T = kFp8Threads, U = kFp8Unroll;
  const int64_t stride = (int64_t)gridDim.x * T * U;
  for (int64_t c0 = (int64_t)blockIdx.x * T * U + threadIdx.x; c0 < total_units; c0 += stride) {
    v4i d[U][2];
    int64_t qo[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + (int64_t)u * T;
      ok[u] = c < total_units;
      int64_t xo;
      if (contiguous) {
        xo = c * 8;
        qo[u] = c * 8;
      } else {
        const uint32_t cc = (uint32_t)c;
        const uint32_t row = cc / units_per_row;
        const uint32_t col = cc - row * units_per_row;
        xo = (int64_t)row * ld_x + col * 8;
        qo[u] = (int64_t)row * ld_q + col * 8;
      }
      d[u][0] = v4i{0, 0, 0, 0};
      d[u][1] = v4i{0, 0, 0, 0};
      if (ok[u]) {
        if (F32) {
          const v4i* p = reinterpret_cast<const v4i*>(static_cast<const float*>(x) + xo);
          d[u][0] = __builtin_nontemporal_load(p);
          d[u][1] = __builtin_nontemporal_load(p + 1);
        } else {
          d[u][0] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(static_cast<const uint16_t*>(x) + xo));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[8];
      if (F32) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) { v[jj] = __int_as_float(d[u][0][jj]); v[4 + jj] = __int_as_float(d[u][1][jj]); }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          v[2 * jj] = bf16_lo_f32(d[u][0][jj]);
          v[2 * jj + 1] = bf16_hi_f32(d[u][0][jj]);
        }
      }
      v2u o;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float y[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) y[jj] = __builtin_amdgcn_fmed3f(v[4 * i + jj] * inv_scale, -448.0f, 448.0f);
        int r = 0;
        r = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], r, false);
        r = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], r, true);
        o[i] = (unsigned)r;
      }
      if (ok[u]) __builtin_nontemporal_store(o, reinterpret_cast<v2u*>(out + qo[u]));
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
// MXFP4 -> bf16: bf16_RNE(e2m1(code) * 2^(s - 127)).  The product has at most 2
// significant bits and lies in bf16's exponent range down to the subnormal 2^-128, so it
// is exact unless it overflows (to +-inf); scale byte 0xFF gives NaN.  One gfx950
// conversion per code byte does the scaling and the rounding.
// CONTIG: codes, scales and output are packed rows (offsets are linear in the quarter
// index); otherwise the row comes from one 32-bit division (quarters < 2^32).
template <bool CONTIG>
__global__ __launch_bounds__(kDqThreads) void dequantize_kernel(
    const uint8_t* __restrict__ codes, int64_t ld_codes, const uint8_t* __restrict__ scales,
    int64_t ld_scales, uint16_t* __restrict__ y, int64_t ld_y, uint32_t blocks_per_row,
    uint32_t total_quarters) {
  // each lane takes kDqUnroll quarters (8 elements each) per pass, loads first
  // the pass counter is 64-bit so that it cannot wrap; quarter indices themselves fit 32 bits
  const uint64_t stride = (uint64_t)gridDim.x * kDqThreads * kDqUnroll;
  for (uint64_t g0 = (uint64_t)blockIdx.x * kDqThreads * kDqUnroll + threadIdx.x; g0 < total_quarters; g0 += stride) {
    unsigned c[kDqUnroll], s[kDqUnroll];
    int64_t yo[kDqUnroll];
    bool ok[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const uint64_t g64 = g0 + (uint64_t)u * kDqThreads;
      ok[u] = g64 < total_quarters;
      const uint32_t g = ok[u] ? (uint32_t)g64 : 0u;
      int64_t co, so;
      if (CONTIG) {
        co = (int64_t)g * 4;
        so = g >> 2;
        yo[u] = (int64_t)g * 8;
      } else {
        const uint32_t b = g >> 2, q = g & 3;
        const uint32_t row = b / blocks_per_row;
        const uint32_t blk = b - row * blocks_per_row;
        co = (int64_t)row * ld_codes + blk * 16 + q * 4;
        so = (int64_t)row * ld_scales + blk;
        yo[u] = (int64_t)row * ld_y + blk * 32 + q * 8;
      }
      c[u] = ok[u] ? *reinterpret_cast<const unsigned*>(codes + co) : 0u;
      s[u] = ok[u] ? scales[so] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      // v_cvt_scalef32_pk_bf16_fp4: the two E2M1 nibbles of byte i (low nibble first) times
      // the binary32 scale, rounded once to bf16.  Checked on the GPU against the exact
      // product for every code byte under every scale byte: exact RNE, the subnormal
      // 2^-127 scale taken as such, overflow to +-inf, -0 kept; a NaN scale (byte 0xFF)
      // gives NaN.
      const unsigned sv = s[u];
      const float sc = sv == 255 ? __uint_as_float(0x7FC00000u) : e8m0_to_f32(sv);
      v4i o;
      o[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], sc, 0));
      o[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], sc, 1));
      o[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], sc, 2));
      o[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], sc, 3));
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


// ---------------------------------------------------------------------------------
// FP8 E4M3 -> bf16 dequantization of statically scaled activations: y = bf16_RNE(
// fl32(e4m3(q) * a_scale)).  v_cvt_pk_f32_fp8 widens two OCP E4M3 bytes exactly to
// binary32 (NaN for S.1111.111); the product is one binary32 multiply; v_cvt_pk_bf16_f32
// rounds to nearest even.  A lane owns 8 consecutive codes of a row per unit.
// CONTIG as in dequantize_kernel (units < 2^32).
template <bool CONTIG>
__global__ __launch_bounds__(kDq8Threads) void dequantize_fp8_kernel(const uint8_t* __restrict__ q, int64_t ld_q,
                                                                    float a_scale, uint16_t* __restrict__ y,
                                                                    int64_t ld_y, uint32_t units_per_row,
                                                                    uint32_t total_units) {
  const uint64_t stride = (uint64_t)gridDim.x * kDq8Threads * kDq8Unroll;
  for (uint64_t g0 = (uint64_t)blockIdx.x * kDq8Threads * kDq8Unroll + threadIdx.x; g0 < total_units; g0 += stride) {
    v2u c[kDq8Unroll];
    int64_t yo[kDq8Unroll];
    bool ok[kDq8Unroll];
#pragma unroll
    for (int u = 0; u < kDq8Unroll; ++u) {
      const uint64_t g64 = g0 + (uint64_t)u * kDq8Threads;
      ok[u] = g64 < total_units;
      const uint32_t g = ok[u] ? (uint32_t)g64 : 0u;
      int64_t qo;
      if (CONTIG) {
        qo = (int64_t)g * 8;
        yo[u] = qo;
      } else {
        const uint32_t row = g / units_per_row;
        const uint32_t col = (g - row * units_per_row) * 8u;
        qo = (int64_t)row * ld_q + col;
        yo[u] = (int64_t)row * ld_y + col;
      }
      c[u] = ok[u] ? *reinterpret_cast<const v2u*>(q + qo) : v2u{0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kDq8Unroll; ++u) {
      v4i o;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int word = (int)c[u][h];
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);   // bytes 0, 1
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);    // bytes 2, 3
        o[2 * h] = (int)pack_bf16x2(lo[0] * a_scale, lo[1] * a_scale);
        o[2 * h + 1] = (int)pack_bf16x2(hi[0] * a_scale, hi[1] * a_scale);
      }
      if (ok[u]) __builtin_nontemporal_store(o, reinterpret_cast<v4i*>(y + yo[u]));
    }
  }
}

}  // namespace

hipError_t launch_quantize_mxfp4(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x,
                                 uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                 bool uos, hipStream_t stream) {
  const int64_t bpr = cols / 32;
  const int64_t total = rows * bpr;
  if (total == 0) return hipSuccess;
  const bool contiguous = ld_x == cols && ld_codes == cols / 2 && ld_scales == bpr;
  const int grid = grid_for(total, kMxBlocksPerIter);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kMxThreads), 0, stream, x, ld_x, codes, ld_codes, scales, ld_scales,
                       (uint32_t)bpr, total);
  };
  auto pick = [&](auto f_tag, auto u_tag) {
    constexpr bool F = decltype(f_tag)::value, R = decltype(u_tag)::value;
    contiguous ? go(mx_quantize_kernel<F, R, true>) : go(mx_quantize_kernel<F, R, false>);
  };
  if (f32)
    uos ? pick(std::true_type{}, std::true_type{}) : pick(std::true_type{}, std::false_type{});
  else
    uos ? pick(std::false_type{}, std::true_type{}) : pick(std::false_type{}, std::false_type{});
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x,
                               float inv_scale, uint8_t* q, int64_t ld_q, hipStream_t stream) {
  const int64_t upr = cols / 8;
  const int64_t total = rows * upr;
  if (total == 0) return hipSuccess;
  const int contiguous = (ld_x == cols && ld_q == cols) ? 1 : 0;
  const int grid = grid_for(total, kFp8Threads * kFp8Unroll);
  if (f32)
    hipLaunchKernelGGL(fp8_quantize_kernel<true>, dim3(grid), dim3(kFp8Threads), 0, stream, x, ld_x, inv_scale,
                       q, ld_q, (uint32_t)upr, total, contiguous);
  else
    hipLaunchKernelGGL(fp8_quantize_kernel<false>, dim3(grid), dim3(kFp8Threads), 0, stream, x, ld_x, inv_scale,
                       q, ld_q, (uint32_t)upr, total, contiguous);
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
  const int64_t total = rows * bpr * 4;   // quarters: below 2^32 (the API bounds rows * cols / 8)
  if (total == 0) return hipSuccess;
  const int grid = grid_for(total, kDqThreads * kDqUnroll);
  const bool contig = ld_codes == cols / 2 && ld_scales == bpr && ld_y == cols;
  hipLaunchKernelGGL(contig ? dequantize_kernel<true> : dequantize_kernel<false>, dim3(grid), dim3(kDqThreads), 0,
                     stream, codes, ld_codes, scales, ld_scales, y, ld_y, (uint32_t)bpr, (uint32_t)total);
  return hipGetLastError();
}

hipError_t launch_dequantize_fp8(const uint8_t* q, int64_t ld_q, float a_scale, int64_t rows, int64_t cols,
                                 uint16_t* y, int64_t ld_y, hipStream_t stream) {
  const int64_t upr = cols / 8;
  const int64_t total = rows * upr;       // below 2^32 (the API bounds rows * cols / 8)
  if (total == 0) return hipSuccess;
  const int grid = grid_for(total, kDq8Threads * kDq8Unroll);
  const bool contig = ld_q == cols && ld_y == cols;
  hipLaunchKernelGGL(contig ? dequantize_fp8_kernel<true> : dequantize_fp8_kernel<false>, dim3(grid),
                     dim3(kDq8Threads), 0, stream, q, ld_q, a_scale, y, ld_y, (uint32_t)upr, (uint32_t)total);
  return hipGetLastError();
}

}  // namespace mxq
