// Fixed block-Hadamard rotation followed by MXFP4 quantization, for gfx950.
//
// Method ("AMD Quark adds native W4A8 mixed-precision for Wan2.2 ...", section "Quark
// quantization pipeline and mixed-precision selection": a fixed Hadamard rotation as the
// transform condition; "Exp 2026-08-22 W4A4 Reference Model", section "Status":
// block-Hadamard with per-group scales): every run of N consecutive elements along K
// becomes x H_N / sqrt(N) (Sylvester H_N, N = 16, 64, 256, so 1/sqrt(N) is a power of
// two), formed in binary32 by the radix-2 butterfly in stage order h = 1, 2, 4, ...: the
// pair (i, i + h) becomes (x_i + x_{i+h}, x_i - x_{i+h}), and the result is scaled by
// 1/sqrt(N).  The rotated binary32 values are then quantized with the MXFP4 rule of
// quantize.hip (OCP or UOS scale byte from the block maximum, E2M1 round-to-nearest-even
// with saturation).  Adds and the final scaling are explicitly rounded (no contraction).
//
// Mapping: one whole 32-element block per lane.  A wave loads 64 consecutive blocks with
// 16 contiguous bytes per lane, so every load instruction moves 1 KB of contiguous input,
// parks them in its own region of LDS and reads them back so that each lane holds one
// block.  Stages h = 1 ... 16 (all of them for N = 16) then stay in the lane; stages
// h = 32, 64, 128 pair the lanes holding blocks b and b ^ (h / 32) through DPP, and the
// block maximum needs no exchange.  Loading one block per lane straight from memory
// (64 bytes per lane per block) costs the address unit more than this LDS round trip.
//
// Built with -fno-slp-vectorize: the SLP vectorizer turns a cross-lane stage's adds into
// vector operations, after which the DPP exchange is no longer folded into the add as an
// operand modifier (one extra move per element and stage).
#include <type_traits>

#include "mxq_device.hpp"
#include "mxq_internal.hpp"

namespace mxq {
namespace {

// 512-thread workgroups, two blocks per lane per pass, one 4 KB (bf16) or 8 KB (binary32)
// LDS region per wave: 73-75 % of HBM for N = 16, 64, 256 on bf16 input (256 or 1024
// threads, one to four blocks per lane, and a region per pass were within 8 % of it)
constexpr int kRotThreads = 512;
constexpr int kRotUnroll = 2;

template <bool F32, int N, bool UOS, bool CONTIG>
__global__ __launch_bounds__(kRotThreads) void mx_quantize_rot_kernel(
    const void* __restrict__ x, int64_t ld_x, uint8_t* __restrict__ codes, int64_t ld_codes,
    uint8_t* __restrict__ scales, int64_t ld_scales, uint32_t blocks_per_row, int64_t total_blocks) {
  static_assert(N == 16 || N == 64 || N == 256, "rotation runs of 16, 64 or 256");
  constexpr float kNorm = N == 16 ? 0.25f : (N == 64 ? 0.125f : 0.0625f);   // 1 / sqrt(N)
  constexpr int WAVES = kRotThreads / 64;
  constexpr int U = kRotUnroll;
  constexpr int RU = F32 ? 8 : 4;                  // 16-byte units per block
  constexpr int RU_SHIFT = F32 ? 3 : 2;
  constexpr int ESZ = F32 ? 4 : 2;
  constexpr int BLOCKS_PER_ITER = kRotThreads * U;
  __shared__ v4i stage[WAVES][64 * RU];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // For N = 256 lane p rotates block p ^ 3 bit2(p) of its group of 8: blocks b ^ 1 and
  // b ^ 2 stay on lanes p ^ 1 and p ^ 2, and block b ^ 4 moves to lane p ^ 7, the DPP
  // half-row mirror (no shifts and select).
  const int slot = N == 256 ? lane ^ (((lane >> 2) & 1) * 3) : lane;
  // Unit c of block b sits at unit c ^ sw(b) of the block's LDS row: the 16-byte writes
  // of 16 consecutive lanes and the block-per-lane reads each cover all 64 banks.
  auto swz = [](int b, int c) { return b * RU + (c ^ (F32 ? ((b >> 1) & 7) : ((b >> 2) & 3))); };
  const int ld_slot = lane >> RU_SHIFT;            // load j fetches unit lane % RU of block j * 64 / RU + ld_slot
  const int ld_unit = lane & (RU - 1);
  const int64_t stride = (int64_t)gridDim.x * BLOCKS_PER_ITER;
  for (int64_t base = (int64_t)blockIdx.x * BLOCKS_PER_ITER; base < total_blocks; base += stride) {
    v4i raw[U][RU];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t wb = base + (int64_t)(u * WAVES + wave) * 64;
      if constexpr (CONTIG) {
        // the wave's 64 blocks are one span; loads past the last block read zero
        const int64_t left = total_blocks - wb;
        const uint32_t nb = left <= 0 ? 0u : (uint32_t)(left < 64 ? left : 64) * (RU * 16);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(static_cast<const char*>(x) + (nb ? wb * (RU * 16) : 0), nb);
#pragma unroll
        for (int j = 0; j < RU; ++j)   // aux 2: non-temporal, the input is read once
          raw[u][j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, j * 1024 + lane * 16, 0, 2));
      } else {
#pragma unroll
        for (int j = 0; j < RU; ++j) {
          const int64_t b = wb + j * (64 / RU) + ld_slot;
          raw[u][j] = v4i{0, 0, 0, 0};
          if (b < total_blocks) {
            const uint32_t bb = (uint32_t)b;
            const uint32_t row = bb / blocks_per_row;
            const uint32_t blk = bb - row * blocks_per_row;
            const int64_t off = (int64_t)row * ld_x * ESZ + (int64_t)blk * (RU * 16) + ld_unit * 16;
            raw[u][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(static_cast<const char*>(x) + off));
          }
        }
      }
    }
    // Each pass's block-per-lane reads follow its own writes.  A wave's LDS operations
    // complete in order, so one region per wave serves every pass; the wavefront-scope
    // fences only keep the compiler from reordering the hand-over.
    float v[U][32];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int j = 0; j < RU; ++j) stage[wave][swz(j * (64 / RU) + ld_slot, ld_unit)] = raw[u][j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int c = 0; c < RU; ++c) {
        const v4i t = stage[wave][swz(slot, c)];
        if (F32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[u][4 * c + i] = __int_as_float(t[i]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {   // bf16 pairs widen exactly (a shift, a mask)
            v[u][8 * c + 2 * i] = bf16_lo_f32(t[i]);
            v[u][8 * c + 2 * i + 1] = bf16_hi_f32(t[i]);
          }
        }
      }
    }
    // stages h = 1 ... 16 inside the lane (runs of 16 for N = 16)
#pragma unroll
    for (int h = 1; h < (N < 32 ? N : 32); h *= 2)
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if ((i & h) == 0) {
            const float a = v[u][i], c = v[u][i + h];
            v[u][i] = __fadd_rn(a, c);
            v[u][i + h] = __fsub_rn(a, c);
          }
    // Stages h = 32, 64, 128 across the lanes holding blocks b and b ^ D, D = h / 32; the
    // lower block keeps the sum.  Both lanes form partner + own', own' = own with its sign
    // flipped in the upper lane: x_i + x_{i+h} (addition commutes) and x_i + (-x_{i+h}),
    // the same binary32 operation as x_i - x_{i+h}.  One add per element and stage with
    // the exchange folded in as its DPP operand.  A DPP instruction waits out two cycles
    // after any write of one of its operands, so each group of 8 flips precedes its adds.
    auto cross = [&](auto d_tag) {
      constexpr int D = decltype(d_tag)::value;
      if constexpr (D < N / 32) {
        constexpr int ctrl = D == 1 ? 0xB1 : (D == 2 ? 0x4E : 0x141);   // quad_perm [1,0,3,2], [2,3,0,1]; row_half_mirror
        const unsigned flip = (slot & D) ? 0x80000000u : 0u;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int g = 0; g < 32; g += 8) {
            float own[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) own[i] = __uint_as_float(__float_as_uint(v[u][g + i]) ^ flip);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float partner = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[u][g + i]), ctrl, 0xF, 0xF, true));
              v[u][g + i] = __fadd_rn(partner, own[i]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
      }
    };
    cross(std::integral_constant<int, 1>{});
    cross(std::integral_constant<int, 2>{});
    cross(std::integral_constant<int, 4>{});
    // scaling by 1/sqrt(N), then MXFP4 of the block (as mx_quantize_kernel)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      unsigned m = 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        v[u][i] = __fmul_rn(v[u][i], kNorm);
        m = max(m, __float_as_uint(v[u][i]) & 0x7FFFFFFFu);
      }
      const unsigned e = m >> 23;
      const unsigned s = UOS ? scale_byte_uos(e, (m & 0x7FFFFFu) > 0x680000u ? 1u : 0u) : scale_byte_from_exp(e);
      const float scale = e8m0_to_f32(s);
      v4i r;
#pragma unroll
      for (int w = 0; w < 4; ++w) {   // byte k of word w: elements 8w + 2k (low nibble), 8w + 2k + 1
        unsigned t = 0;
        t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, v[u][8 * w + 0], v[u][8 * w + 1], scale, 0);
        t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, v[u][8 * w + 2], v[u][8 * w + 3], scale, 1);
        t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, v[u][8 * w + 4], v[u][8 * w + 5], scale, 2);
        t = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(t, v[u][8 * w + 6], v[u][8 * w + 7], scale, 3);
        r[w] = (int)t;
      }
      const int64_t wb = base + (int64_t)(u * WAVES + wave) * 64;
      if constexpr (CONTIG) {
        // stores past the last block are dropped by the buffer range check
        const int64_t left = total_blocks - wb;
        const uint32_t nb = left <= 0 ? 0u : (uint32_t)(left < 64 ? left : 64);
        // (a wave past the last block gets an empty range at the buffer's start)
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes + (nb ? wb * 16 : 0), nb * 16);
        const __amdgpu_buffer_rsrc_t rsc = make_rsrc(scales + (nb ? wb : 0), nb);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, r), rc, slot * 16, 0, 2);
        __builtin_amdgcn_raw_buffer_store_b8((unsigned char)s, rsc, slot, 0, 2);
      } else {
        const int64_t b = wb + slot;
        if (b < total_blocks) {
          const uint32_t bb = (uint32_t)b;
          const uint32_t row = bb / blocks_per_row;
          const uint32_t blk = bb - row * blocks_per_row;
          __builtin_nontemporal_store(r, reinterpret_cast<v4i*>(codes + (int64_t)row * ld_codes + blk * 16));
          scales[(int64_t)row * ld_scales + blk] = (uint8_t)s;
        }
      }
    }
  }
}

}  // namespace

// A run never straddles a row (the API requires K % N == 0) and starts at a multiple of
// N / 32 blocks, so its blocks sit on lanes b, b ^ 1, ... of one group of a wave.
hipError_t launch_quantize_mxfp4_rotated(const void* x, bool f32, int64_t rows, int64_t cols, int64_t ld_x, int n,
                                         uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                         bool uos, hipStream_t stream) {
  const int64_t bpr = cols / 32;
  const int64_t total = rows * bpr;
  if (total == 0) return hipSuccess;
  const bool contiguous = ld_x == cols && ld_codes == cols / 2 && ld_scales == bpr;
  constexpr int64_t per_block = (int64_t)kRotThreads * kRotUnroll;
  int64_t g = (total + per_block - 1) / per_block;
  if (g > 256 * 64) g = 256 * 64;   // enough resident waves to cover HBM latency; the rest loop
  const int grid = (int)g;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kRotThreads), 0, stream, x, ld_x, codes, ld_codes, scales,
                       ld_scales, (uint32_t)bpr, total);
  };
  auto pick_layout = [&](auto f32_tag, auto n_tag, auto uos_tag) {
    constexpr bool F = decltype(f32_tag)::value;
    constexpr int NN = decltype(n_tag)::value;
    constexpr bool R = decltype(uos_tag)::value;
    contiguous ? go(mx_quantize_rot_kernel<F, NN, R, true>) : go(mx_quantize_rot_kernel<F, NN, R, false>);
  };
  auto pick_rule = [&](auto f32_tag, auto n_tag) {
    uos ? pick_layout(f32_tag, n_tag, std::true_type{}) : pick_layout(f32_tag, n_tag, std::false_type{});
  };
  auto pick_n = [&](auto f32_tag) {
    if (n == 16)
      pick_rule(f32_tag, std::integral_constant<int, 16>{});
    else if (n == 64)
      pick_rule(f32_tag, std::integral_constant<int, 64>{});
    else
      pick_rule(f32_tag, std::integral_constant<int, 256>{});
  };
  f32 ? pick_n(std::true_type{}) : pick_n(std::false_type{});
  return hipGetLastError();
}

}  // namespace mxq
