// Device-side helpers shared by the gfx950 kernels: vector types, buffer resources,
// quad (4-lane) reductions and bf16 packing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef unsigned short v2h __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Raw buffer resource over [base, base + bytes): loads past `bytes` return zero, which
// the kernels use to zero-fill ragged tiles without branches.  Word 3 is the gfx9
// raw-buffer format (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Max over the 4 lanes of a quad (lanes 4q..4q+3) with DPP quad permutations.
__device__ __forceinline__ unsigned quad_max_u32(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));  // lane ^ 1
  v = max(v, (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));  // lane ^ 2
  return v;
}

// The low / high bf16 of a packed pair as binary32 (exact: the bf16 bits become the top
// half of the binary32 word).
__device__ __forceinline__ float bf16_lo_f32(int pair) { return __uint_as_float((unsigned)pair << 16); }
__device__ __forceinline__ float bf16_hi_f32(int pair) { return __uint_as_float((unsigned)pair & 0xFFFF0000u); }

// Two floats -> packed bf16x2 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, v);
}

// The E8M0 scale 2^(s - 127) as a binary32: exponent field s, or the subnormal 2^-127
// for s == 0.
__device__ __forceinline__ float e8m0_to_f32(unsigned s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// MXFP4 scale byte from the biased exponent field e of the block maximum: the OCP rule
// s = max(e - 2, 0); non-finite blocks (e == 255) get the E8M0 NaN.
__device__ __forceinline__ unsigned scale_byte_from_exp(unsigned e) {
  return e == 255u ? 255u : (e > 2u ? e - 2u : 0u);
}

// The UOS rule: one more when the significand of a normal maximum exceeds 1.8125
// (bump = 1), floored at 0 like the OCP rule.
__device__ __forceinline__ unsigned scale_byte_uos(unsigned e, unsigned bump) {
  const unsigned t = e + (e != 0u ? bump : 0u);
  return e == 255u ? 255u : (t > 2u ? t - 2u : 0u);
}

}  // namespace mxq
