// Block-scaled MFMA GEMMs for gfx950: W4A4 (MXFP4 x MXFP4), W4A8 (MXFP4 weights x FP8
// E4M3 activations) and the bf16 reference, all out = A * W^T with fp32 accumulation and
// a bf16 (round to nearest even) epilogue.
//
// What is computed ("AMD Quark adds native W4A8 mixed-precision for Wan2.2 ...", section
// "Quark quantization pipeline and mixed-precision selection"; "AMD Quark: 1.92x faster
// FLUX.1-dev ...", section "MXFP4 quantization for diffusion models": the GEMM consumes
// MXFP4 directly with no dequantization phase; "Exp 2026-08-22 W4A4 Reference Model",
// section "Status": a linear per-group scale factors out of the group's partial sum):
//   W4A4: out[m,n] = sum_b 2^(SA[m,b]+SW[n,b]-254) * sum_i e2m1(QA[m,32b+i]) e2m1(QW[n,32b+i])
//   W4A8: out[m,n] = s_a * sum_b 2^(SW[n,b]-127) * sum_i e4m3(QA8[m,32b+i]) e2m1(QW[n,32b+i])
// The per-block scales are applied inside v_mfma_scale_f32_32x32x64_f8f6f4, which takes
// one E8M0 byte per (row, 32-K block) per operand, so no value is ever dequantized.
//
// Tiling (one workgroup = 4 waves = a 256 (m) x 256 (n) output tile; one wave = 128 x 128):
//  * The weight tile is the MFMA A operand and the activation tile the B operand, so
//    every lane finishes holding 4 consecutive output columns of one row (8-byte stores).
//  * K advances in windows of 128 bytes per row (256 fp4 / 128 fp8 / 64 bf16 values).
//    Each window is staged global -> registers -> LDS, double buffered (2 x 64 KB), with
//    16-byte chunks XOR-swizzled by row so MFMA fragment reads are bank-conflict free
//    (the fast path streams global -> LDS directly with buffer_load ... lds).
//  * Inside a window the MFMA K-slots are assigned so that lane group g (lanes 32g..32g+31)
//    at MFMA step t holds K-block 4g+t (fp4): a lane reads contiguous 16-byte chunks and
//    one 32-bit word holds its four scale bytes, selected by op_sel = t.  Any assignment
//    is valid as long as both operands and the scales agree; the sum over K is the same.
//  * FP8 operands occupy the MFMA K range in two halves (per lane: 16 bytes from the low
//    half, 16 from the high half), so W4A8 reads two 16-byte chunks per fragment.
//  * Workgroups are renumbered so that each XCD (dispatched round-robin) walks a
//    contiguous run of tiles, grouped 4 m-tiles wide, keeping panels shared in its L2.
//  * Ragged M/N/K tails are zero-filled by buffer-load range checks and masked stores.
//  * The bf16 reference (gemm_bf16_kernel) uses 16 x 16 x 32 MFMAs in eight waves (two per
//    SIMD, 128 x 64 per wave): under the chip's power limit that shape sustains more
//    MFMA throughput on real data than 32 x 32 x 16.
//  * gemm_w4a4_fused8_kernel takes unquantized activations and quantizes each activation
//    tile into LDS inside the GEMM, bit-identically to the separate quantizer.
#include <type_traits>
#include <utility>

#include "mxq_device.hpp"
#include "mxq_internal.hpp"


namespace mxq {
namespace {

constexpr int BM = 256;   // activation rows per workgroup
constexpr int BN = 256;   // weight rows per workgroup
constexpr int NT = 256;   // threads per workgroup
constexpr int GROUP_M = 4;
constexpr int64_t kStreamOutMaxK = 8192;   // largest K whose output stores are non-temporal

template <int MODE> struct Cfg;
// Geometry of the generic (register-staged) kernel: bytes per row per window of the
// activation / weight tiles, MFMA steps per window, K elements per window.
template <> struct Cfg<GEMM_W4A4> {
  static constexpr int A_RB = 128, W_RB = 128, STEPS = 4, K_WIN = 256;
};
template <> struct Cfg<GEMM_W4A8> {
  static constexpr int A_RB = 128, W_RB = 64, STEPS = 2, K_WIN = 128;
};
template <> struct Cfg<GEMM_BF16> {
  static constexpr int A_RB = 128, W_RB = 128, STEPS = 4, K_WIN = 64;
};

// Fast-path geometry of gemm_fast_kernel (the scaled modes).  A_RB / W_RB: bytes per row
// per K-window for the activation / weight tile (128 bytes: whole cache lines per row);
// STEPS: 32x32 MFMA steps per window; NS: depth of both tile rings in LDS (a window's
// loads get about NS-1 windows of compute to land); SC_WIN: scale bytes per row per
// window.  Lane group g at step t holds K-chunk g * STEPS + t of the weight row (and of
// the activation row for FP4 activations).  The bf16 reference has its own kernel
// (gemm_bf16_kernel) over windows of K_WIN elements.
template <int MODE> struct Fast;
template <> struct Fast<GEMM_W4A4> {
  static constexpr int A_RB = 128, W_RB = 128, STEPS = 4, K_WIN = 256, NS = 2, SC_WIN = 8;
};
template <> struct Fast<GEMM_W4A8> {
  static constexpr int A_RB = 128, W_RB = 64, STEPS = 2, K_WIN = 128, NS = 3, SC_WIN = 4;
};
template <> struct Fast<GEMM_BF16> {
  static constexpr int K_WIN = 64;
};

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt <= 0, expcnt unconstrained
constexpr int waitcnt_vm(int vm) { return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4); }

// Workgroup barrier for the LDS stage hand-over.  The caller has already waited (s_waitcnt)
// for exactly the loads that must have landed; __syncthreads() would add a release fence
// that drains every outstanding load, including the later stages still in flight.  The
// empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Column of byte `col` (0..31) of a row of a 32-byte-per-row scale chunk in LDS, for a row
// whose index within its 32-row line is r: rows with bit 2 set hold their 16-byte halves
// swapped (the chunk loads place them so).
__device__ __forceinline__ uint32_t sc_col(uint32_t col, uint32_t r) { return col ^ (16u * ((r >> 2) & 1u)); }

}  // namespace

// Kernel arguments of every GEMM kernel here (named, so that the scaled-GEMM object built
// from this file with MXQ_GEMM_SCALED_OBJECT shares the type with its launcher).
struct Params {
  const uint8_t* a;
  const uint8_t* a_scales;
  const uint8_t* w;
  const uint8_t* w_scales;
  uint16_t* out;
  int64_t ld_out;
  int M, N;
  uint32_t a_row_bytes, w_row_bytes, scale_row_bytes;
  int nwin, tiles_m, tiles_n;
  float a_scale;
  int vec_store;   // 8-byte output stores allowed (pitch and base)
  int vec16;       // 16-byte output stores allowed
  int scale_dword_ok;
  int stream_out;  // staged output stores carry the non-temporal hint
};

namespace {

// LDS swizzles.  The LDS serves a ds_read_b128 16 lanes at a time over 64 4-byte banks
// (256 bytes); fragment reads have 16 consecutive lanes on 16 consecutive rows at one
// logical chunk, so the 16-byte slot of chunk c in row r is c ^ f(r) with f distinct
// over the rows that share banks: 128-byte rows pair up per 256 bytes (f = (r>>1)&7),
// 64-byte rows quarter it (f = (r>>2)&3).
__device__ __forceinline__ uint32_t swz128(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row >> 1) & 7u)) << 4);
}
__device__ __forceinline__ uint32_t swz64(uint32_t row, uint32_t chunk) {
  return row * 64u + ((chunk ^ ((row >> 2) & 3u)) << 4);
}

template <int RB>
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  if constexpr (RB == 128)
    return swz128(row, chunk);
  else
    return swz64(row, chunk);
}

__device__ __forceinline__ v8i widen(v4i x) { return v8i{x[0], x[1], x[2], x[3], 0, 0, 0, 0}; }
__device__ __forceinline__ v8i cat(v4i x, v4i y) { return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]}; }

// Four scale bytes of one row starting at byte `col`; bytes past the row read as 0
// (a finite 2^-127 multiplying zero-filled data).
__device__ __forceinline__ uint32_t load_scale4(__amdgpu_buffer_rsrc_t r, uint32_t row_off, uint32_t col,
                                                uint32_t row_bytes, int dword_ok) {
  if (dword_ok) {
    const uint32_t off = (col + 4u <= row_bytes) ? row_off + col : 0x80000000u;
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  uint32_t v = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t off = (col + b < row_bytes) ? row_off + col + b : 0x80000000u;
    v |= ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0) & 0xFFu) << (8 * b);
  }
  return v;
}

template <int MODE, int T>
__device__ __forceinline__ void mfma_step(v16f (&acc)[4][4], const uint8_t* lds_a, const uint8_t* lds_w,
                                          uint32_t wm, uint32_t wn, uint32_t lane, const uint32_t (&scw)[4],
                                          const uint32_t (&sca)[4]) {
  const uint32_t g = lane >> 5, r32 = lane & 31;
  if constexpr (MODE == GEMM_W4A4) {
    v4i wf[4], af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wf[i] = *reinterpret_cast<const v4i*>(lds_w + swz128(wn * 128 + 32 * i + r32, 4 * g + T));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      af[j] = *reinterpret_cast<const v4i*>(lds_a + swz128(wm * 128 + 32 * j + r32, 4 * g + T));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(wf[i]), widen(af[j]), acc[i][j], 4, 4, T,
                                                                    (int)scw[i], T, (int)sca[j]);
  } else if constexpr (MODE == GEMM_W4A8) {
    v4i wf[4], alo[4], ahi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wf[i] = *reinterpret_cast<const v4i*>(lds_w + swz64(wn * 128 + 32 * i + r32, 2 * g + T));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t row = wm * 128 + 32 * j + r32;
      alo[j] = *reinterpret_cast<const v4i*>(lds_a + swz128(row, 2 * T + g));
      ahi[j] = *reinterpret_cast<const v4i*>(lds_a + swz128(row, 4 + 2 * T + g));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(wf[i]), cat(alo[j], ahi[j]), acc[i][j], 4,
                                                                    0, T, (int)scw[i], 0, 127);
  } else {
    v4i wf[4], af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wf[i] = *reinterpret_cast<const v4i*>(lds_w + swz128(wn * 128 + 32 * i + r32, 4 * g + T));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      af[j] = *reinterpret_cast<const v4i*>(lds_a + swz128(wm * 128 + 32 * j + r32, 4 * g + T));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wf[i]),
                                                            __builtin_bit_cast(bf16x8, af[j]), acc[i][j], 0, 0, 0);
  }
}

template <int MODE>
__global__ __launch_bounds__(NT, 1) void gemm_generic_kernel(Params p) {
  using C = Cfg<MODE>;
  constexpr uint32_t A_TILE = BM * C::A_RB;
  constexpr uint32_t W_TILE = BN * C::W_RB;
  constexpr uint32_t BUF = A_TILE + W_TILE;
  constexpr int A_CH = A_TILE / 16 / NT;   // 16-byte chunks per thread per window
  constexpr int W_CH = W_TILE / 16 / NT;
  constexpr int A_CPR = C::A_RB / 16;      // chunks per row
  constexpr int W_CPR = C::W_RB / 16;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * BUF];

  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t wm = wave & 1, wn = wave >> 1;

  // ---- tile order: contiguous run per XCD, grouped GROUP_M m-tiles wide ----
  const int nt = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int q8 = nt >> 3, r8 = nt & 7;
  const int seq = xcd * q8 + min(xcd, r8) + local;
  const int group = seq / (GROUP_M * p.tiles_n);
  const int first_m = group * GROUP_M;
  const int gm = min(GROUP_M, p.tiles_m - first_m);
  const int in_group = seq - group * GROUP_M * p.tiles_n;
  const int tm = first_m + in_group % gm, tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const uint32_t rows_a = (uint32_t)min(BM, p.M - m0), rows_w = (uint32_t)min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.a_row_bytes, rows_a * p.a_row_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w + (int64_t)n0 * p.w_row_bytes, rows_w * p.w_row_bytes);

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  if (p.nwin > 0) {
    // per-thread staging geometry (fixed across windows)
    const uint32_t a_c = tid % A_CPR, a_r = tid / A_CPR;
    const uint32_t w_c = tid % W_CPR, w_r = tid / W_CPR;
    constexpr uint32_t A_RSTEP = NT / A_CPR, W_RSTEP = NT / W_CPR;

    // scale planes (unused by the bf16 reference: zero-length resources)
    const bool has_ws = MODE != GEMM_BF16, has_as = MODE == GEMM_W4A4;
    const __amdgpu_buffer_rsrc_t rsw =
        make_rsrc(has_ws ? p.w_scales + (int64_t)n0 * p.scale_row_bytes : p.w, has_ws ? rows_w * p.scale_row_bytes : 0);
    const __amdgpu_buffer_rsrc_t rsa =
        make_rsrc(has_as ? p.a_scales + (int64_t)m0 * p.scale_row_bytes : p.a, has_as ? rows_a * p.scale_row_bytes : 0);
    uint32_t sa_off[4], sw_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sw_off[i] = (wn * 128 + 32 * i + (lane & 31)) * p.scale_row_bytes;
      sa_off[i] = (wm * 128 + 32 * i + (lane & 31)) * p.scale_row_bytes;
    }

    v4i sta[A_CH], stw[W_CH];
    uint32_t scw[4] = {0, 0, 0, 0}, sca[4] = {0, 0, 0, 0}, scw_n[4] = {0, 0, 0, 0}, sca_n[4] = {0, 0, 0, 0};

    auto load_window = [&](int w) {
      const uint32_t abase = (uint32_t)w * C::A_RB + a_c * 16;
      const bool a_in = abase + 16 <= p.a_row_bytes;
#pragma unroll
      for (int i = 0; i < A_CH; ++i) {
        const uint32_t off = a_in ? (a_r + i * A_RSTEP) * p.a_row_bytes + abase : 0x80000000u;
        sta[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      }
      const uint32_t wbase = (uint32_t)w * C::W_RB + w_c * 16;
      const bool w_in = wbase + 16 <= p.w_row_bytes;
#pragma unroll
      for (int i = 0; i < W_CH; ++i) {
        const uint32_t off = w_in ? (w_r + i * W_RSTEP) * p.w_row_bytes + wbase : 0x80000000u;
        stw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
      }
      if constexpr (MODE == GEMM_W4A4) {
        const uint32_t col = (uint32_t)w * 8 + 4 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i) scw_n[i] = load_scale4(rsw, sw_off[i], col, p.scale_row_bytes, p.scale_dword_ok);
#pragma unroll
        for (int j = 0; j < 4; ++j) sca_n[j] = load_scale4(rsa, sa_off[j], col, p.scale_row_bytes, p.scale_dword_ok);
      } else if constexpr (MODE == GEMM_W4A8) {
        const uint32_t col = (uint32_t)w * 4;
        const uint32_t sh = 16 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          scw_n[i] = load_scale4(rsw, sw_off[i], col, p.scale_row_bytes, p.scale_dword_ok) >> sh;
      }
    };
    auto store_window = [&](uint32_t buf) {
      uint8_t* la = lds + buf;
      uint8_t* lw = lds + buf + A_TILE;
#pragma unroll
      for (int i = 0; i < A_CH; ++i) *reinterpret_cast<v4i*>(la + swz128(a_r + i * A_RSTEP, a_c)) = sta[i];
#pragma unroll
      for (int i = 0; i < W_CH; ++i) {
        if constexpr (C::W_RB == 128)
          *reinterpret_cast<v4i*>(lw + swz128(w_r + i * W_RSTEP, w_c)) = stw[i];
        else
          *reinterpret_cast<v4i*>(lw + swz64(w_r + i * W_RSTEP, w_c)) = stw[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        scw[i] = scw_n[i];
        sca[i] = sca_n[i];
      }
    };

    load_window(0);
    store_window(0);
    __syncthreads();
    if (p.nwin > 1) load_window(1);

    for (int w = 0; w < p.nwin; ++w) {
      const uint8_t* la = lds + (w & 1) * BUF;
      const uint8_t* lw = la + A_TILE;
      mfma_step<MODE, 0>(acc, la, lw, wm, wn, lane, scw, sca);
      mfma_step<MODE, 1>(acc, la, lw, wm, wn, lane, scw, sca);
      if constexpr (C::STEPS == 4) {
        mfma_step<MODE, 2>(acc, la, lw, wm, wn, lane, scw, sca);
        mfma_step<MODE, 3>(acc, la, lw, wm, wn, lane, scw, sca);
      }
      if (w + 1 < p.nwin) {
        store_window(((w + 1) & 1) * BUF);
        if (w + 2 < p.nwin) load_window(w + 2);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: fp32 -> bf16 (RNE), lane owns 4 consecutive columns per store ----
  const uint32_t r32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + (int)(wm * 128 + 32 * j + r32);
    if (m >= p.M) continue;
    uint16_t* orow = p.out + (int64_t)m * p.ld_out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int n = n0 + (int)(wn * 128 + 32 * i + 8 * pp + 4 * g);
        float v0 = acc[i][j][4 * pp + 0], v1 = acc[i][j][4 * pp + 1];
        float v2 = acc[i][j][4 * pp + 2], v3 = acc[i][j][4 * pp + 3];
        if constexpr (MODE == GEMM_W4A8) {
          v0 *= p.a_scale;
          v1 *= p.a_scale;
          v2 *= p.a_scale;
          v3 *= p.a_scale;
        }
        const unsigned lo = pack_bf16x2(v0, v1), hi = pack_bf16x2(v2, v3);
        if (p.vec_store && n + 4 <= p.N) {
          *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
        } else {
          const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < p.N) orow[n + e] = h[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Fast path: K is a whole number of windows, and scale rows are 16-byte multiples on
// 16-byte aligned planes (every workload shape).  Tiles stream global -> LDS with
// buffer_load ... lds (no staging registers); each wave issues whole 1 KB LDS lines whose
// lanes fetch the chunk the XOR swizzle places there.  One barrier per window; the next
// window's loads and its first fragment reads are issued under the current window's last
// MFMA step.

// buffer_load_dwordx4 ... lds: 16 bytes per lane into LDS at `lds_line` + 16 * lane
__device__ __forceinline__ void load_line_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds_line, uint32_t voff,
                                                 uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_line, 16, voff, soff, 0, 0);
}

// Fragments of MFMA step t from one LDS stage.  Lane group g (lanes 32g..32g+31) at step t
// holds K-chunk g * STEPS + t of its weight row (one 32-element FP4 block) and the same
// chunk of its FP4 activation row; FP8 activation rows give each lane
// the chunks 2t+g and 4+2t+g that the FP8 operand layout pairs with those FP4 blocks.
//
// `after(k)` runs after the k-th read (k = 0 .. 7, or 11 for W4A8).  LDS-DMA loads issued
// from it land in program order between the reads: the compiler cannot move a read past a
// DMA that may write the same LDS array, so source order is the only way to interleave.
template <int MODE, class After>
__device__ __forceinline__ void read_frags(v4i (&f)[12], const uint8_t* la, const uint8_t* lw, uint32_t wm, uint32_t wn,
                                           uint32_t lane, int t, After&& after) {
  using F = Fast<MODE>;
  const uint32_t g = lane >> 5, r32 = lane & 31;
  const uint32_t chunk = g * F::STEPS + t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = *reinterpret_cast<const v4i*>(lw + swz<F::W_RB>(wn * 128 + 32 * i + r32, chunk));
    after(i);
  }
  if constexpr (MODE == GEMM_W4A8) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t row = wm * 128 + 32 * j + r32;
      f[4 + j] = *reinterpret_cast<const v4i*>(la + swz128(row, 2 * t + g));
      after(4 + 2 * j);
      f[8 + j] = *reinterpret_cast<const v4i*>(la + swz128(row, 4 + 2 * t + g));
      after(5 + 2 * j);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f[4 + j] = *reinterpret_cast<const v4i*>(la + swz<F::A_RB>(wm * 128 + 32 * j + r32, chunk));
      after(4 + j);
    }
  }
}

template <int MODE>
__device__ __forceinline__ void read_frags(v4i (&f)[12], const uint8_t* la, const uint8_t* lw, uint32_t wm, uint32_t wn,
                                           uint32_t lane, int t) {
  read_frags<MODE>(f, la, lw, wm, wn, lane, t, [](int) {});
}

// number of the n DMA loads spread over rd reads that go out right after read k
constexpr int dma_after(int k, int n, int rd) { return (k + 1) * n / rd - k * n / rd; }

template <int MODE, int T>
__device__ __forceinline__ void mfma16(v16f (&acc)[4][4], const v4i (&f)[12], const uint32_t (&scw)[4],
                                       const uint32_t (&sca)[4]) {
  static_assert(MODE == GEMM_W4A4 || MODE == GEMM_W4A8, "scaled modes only");
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MODE == GEMM_W4A4)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f[i]), widen(f[4 + j]), acc[i][j], 4, 4, T,
                                                                    (int)scw[i], T, (int)sca[j]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f[i]), cat(f[4 + j], f[8 + j]), acc[i][j],
                                                                    4, 0, T, (int)scw[i], 0, 127);
    }
}

// Epilogue of tiles the staged path does not take (a partial column tile or an output
// that is not 16-byte aligned): a lane owns 4 consecutive columns per store.
template <int MODE>
__device__ __forceinline__ void store_partial_tile(const Params& p, const v16f (&acc)[4][4], uint32_t lane, uint32_t wm,
                                                   uint32_t wn, int m0, int n0) {
  const uint32_t r32 = lane & 31, g = lane >> 5;
  const bool full = p.vec_store && m0 + BM <= p.M && n0 + BN <= p.N;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + (int)(wm * 128 + 32 * j + r32);
    uint16_t* orow = p.out + (int64_t)min(m, p.M - 1) * p.ld_out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int n = n0 + (int)(wn * 128 + 32 * i + 8 * pp + 4 * g);
        float v0 = acc[i][j][4 * pp + 0], v1 = acc[i][j][4 * pp + 1];
        float v2 = acc[i][j][4 * pp + 2], v3 = acc[i][j][4 * pp + 3];
        if constexpr (MODE == GEMM_W4A8) {
          v0 *= p.a_scale;
          v1 *= p.a_scale;
          v2 *= p.a_scale;
          v3 *= p.a_scale;
        }
        const unsigned lo = pack_bf16x2(v0, v1), hi = pack_bf16x2(v2, v3);
        if (full) {
          *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
        } else if (m < p.M) {
          if (p.vec_store && n + 4 <= p.N) {
            *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
          } else {
            if (n + 0 < p.N) orow[n + 0] = (uint16_t)lo;
            if (n + 1 < p.N) orow[n + 1] = (uint16_t)(lo >> 16);
            if (n + 2 < p.N) orow[n + 2] = (uint16_t)hi;
            if (n + 3 < p.N) orow[n + 3] = (uint16_t)(hi >> 16);
          }
        }
      }
    }
  }
}

// STREAM: the staged output stores carry the non-temporal hint (Params::stream_out).
template <int MODE, bool STREAM>
__global__ __launch_bounds__(NT, 1) void gemm_fast_kernel(Params p) {
  using C = Fast<MODE>;
  constexpr uint32_t A_TILE = BM * C::A_RB;
  constexpr uint32_t W_TILE = BN * C::W_RB;
  constexpr int A_LINES = A_TILE / 1024 / 4;   // 1 KB LDS lines per wave per window
  constexpr int W_LINES = W_TILE / 1024 / 4;
  constexpr int A_ROWS_PER_LINE = 1024 / C::A_RB;
  constexpr int W_ROWS_PER_LINE = 1024 / C::W_RB;
  static_assert(MODE != GEMM_BF16, "the bf16 reference runs gemm_bf16_kernel");
  // Window w+NS's activation tile goes out at the hand-over of window w into the slot it
  // releases, its weight tile under the next window's step 0.
  constexpr int NS = C::NS;                    // windows issued ahead by the prologue + 1
  constexpr uint32_t W_BASE = NS * A_TILE, SC_BASE = NS * A_TILE + NS * W_TILE;
  // Scales travel in chunks of SC_ROW bytes per row (CW windows) through a two-slot ring
  // beside the tile stages: a load instruction costs the memory pipeline per cache line
  // touched, so a few bytes per row per window would cost as much as the tiles themselves.
  // A slot holds the weight rows' chunk, then (W4A4) the activation rows'.
  constexpr uint32_t SC_WIN = C::SC_WIN;       // scale bytes per row per window
  constexpr bool HAS_SC = SC_WIN > 0;
  constexpr uint32_t SC_ROW = 32;
  constexpr int CW = HAS_SC ? (int)(SC_ROW / SC_WIN) : 1;
  constexpr uint32_t SC_ROWS = HAS_SC ? BN + (MODE == GEMM_W4A4 ? BM : 0) : 0;
  constexpr uint32_t SLOT = SC_ROWS * SC_ROW;
  constexpr int SC_LINES = (int)(SLOT / 1024 / 4);   // 1 KB lines (32 rows) per wave per chunk
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SC_BASE + 2 * SLOT];

  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const uint32_t wm = wave & 1, wn = wave >> 1;

  const int nt = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int q8 = nt >> 3, r8 = nt & 7;
  const int seq = xcd * q8 + min(xcd, r8) + local;
  const int group = seq / (GROUP_M * p.tiles_n);
  const int first_m = group * GROUP_M;
  const int gm = min(GROUP_M, p.tiles_m - first_m);
  const int in_group = seq - group * GROUP_M * p.tiles_n;
  const int tm = first_m + in_group % gm, tn = in_group / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  constexpr bool has_as = MODE == GEMM_W4A4;
  const uint32_t rows_a = (uint32_t)min(BM, p.M - m0), rows_w = (uint32_t)min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.a_row_bytes, rows_a * p.a_row_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w + (int64_t)n0 * p.w_row_bytes, rows_w * p.w_row_bytes);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(p.w_scales + (int64_t)n0 * p.scale_row_bytes, rows_w * p.scale_row_bytes);
  const __amdgpu_buffer_rsrc_t rsa =
      make_rsrc(has_as ? p.a_scales + (int64_t)m0 * p.scale_row_bytes : p.a, has_as ? rows_a * p.scale_row_bytes : 0);

  // Lane geometry of the direct-to-LDS tile loads: LDS line q holds rows
  // [q * ROWS_PER_LINE, ...); lane i lands at byte 16 i of the line, i.e. in row i / CPR at
  // slot i % CPR, and fetches the chunk the swizzle maps there.  With 128-byte rows the
  // swizzle term (r>>1)&7 depends on the line's parity: one offset for even lines, one
  // for odd lines.
  constexpr uint32_t A_CPR = C::A_RB / 16, W_CPR = C::W_RB / 16;
  auto dma_voffs = [&](uint32_t cpr, uint32_t row_bytes, uint32_t& even, uint32_t& odd) {
    const uint32_t row = lane / cpr, slot = lane % cpr;
    if (cpr == 8) {                       // 128-byte rows: 8 per line, term (r>>1)&7
      even = row * row_bytes + ((slot ^ ((row >> 1) & 7u)) * 16);
      odd = row * row_bytes + ((slot ^ (((8u + row) >> 1) & 7u)) * 16);
    } else {                              // 64-byte rows: 16 per line, term (r>>2)&3
      even = odd = row * row_bytes + ((slot ^ ((row >> 2) & 3u)) * 16);
    }
  };
  uint32_t a_voff0, a_voff1, w_voff0, w_voff1;
  dma_voffs(A_CPR, p.a_row_bytes, a_voff0, a_voff1);
  dma_voffs(W_CPR, p.w_row_bytes, w_voff0, w_voff1);
  // scale chunk lines: lane i lands in half i & 1 of row i / 2 of the line; rows with bit 2
  // set hold their two 16-byte halves swapped (sc_col), which halves the bank conflicts of
  // the 4-byte scale reads (32 lanes on 32 rows 32 bytes apart)
  const uint32_t sc_voff = (lane >> 1) * p.scale_row_bytes + (((lane & 1) ^ ((lane >> 3) & 1)) * 16);

  // A window's tile loads in two parts, issued under different MFMA steps so that the
  // four waves never queue a whole window of DMA at once: part 0 = activation tile,
  // part 1 = weight tile.  Window w lives in ring slot w mod NS.
  auto a_at = [&](uint32_t sl) { return lds + sl * A_TILE; };
  auto w_at = [&](uint32_t sl) { return lds + W_BASE + sl * W_TILE; };
  // one line of window w's tile into ring slot sl
  auto issue_line = [&](uint32_t sl, int w, auto part_tag, int j) {
    constexpr int PART = decltype(part_tag)::value;
    if constexpr (PART == 0) {
      const uint32_t line = wave * A_LINES + j;
      load_line_to_lds(ra, a_at(sl) + line * 1024, (line & 1) ? a_voff1 : a_voff0,
                       (uint32_t)w * C::A_RB + line * A_ROWS_PER_LINE * p.a_row_bytes);
    } else {
      const uint32_t line = wave * W_LINES + j;
      load_line_to_lds(rw, w_at(sl) + line * 1024, (line & 1) ? w_voff1 : w_voff0,
                       (uint32_t)w * C::W_RB + line * W_ROWS_PER_LINE * p.w_row_bytes);
    }
  };
  auto issue_loads = [&](int w) {
#pragma unroll
    for (int j = 0; j < A_LINES; ++j) issue_line((uint32_t)w % NS, w, std::integral_constant<int, 0>{}, j);
#pragma unroll
    for (int j = 0; j < W_LINES; ++j) issue_line((uint32_t)w % NS, w, std::integral_constant<int, 1>{}, j);
  };
  // scale chunk c (windows c*CW ..) into scale slot c & 1
  const int nchunks = (p.nwin + CW - 1) / CW;
  auto issue_chunk = [&](int c) {
    uint8_t* slot = lds + SC_BASE + (uint32_t)(c & 1) * SLOT;
#pragma unroll
    for (int j = 0; j < SC_LINES; ++j) {
      const uint32_t line = wave * SC_LINES + j;
      const bool is_w = line < BN / 32;
      const uint32_t row0 = (is_w ? line : line - BN / 32) * 32;
      load_line_to_lds(is_w ? rsw : rsa, slot + line * 1024, sc_voff, (uint32_t)c * SC_ROW + row0 * p.scale_row_bytes);
    }
  };
  // Chunk c+1 goes out at the start of window c*CW (c >= 1; chunk 1 in the prologue): the
  // barrier that ended window c*CW - 1 follows every wave's last read of chunk c-1, the
  // slot's previous occupant, and issuing ahead of the window's pending tile loads keeps
  // the chunk older than every tile load the hand-over waits for.
  auto chunk_due = [&](int w) { return w >= CW && w % CW == 0 && w / CW + 1 < nchunks; };
  // this lane's scale bytes for window w: W rows (4 n-fragments), A rows (4 m-fragments);
  // byte t is the block of MFMA step t (op_sel t).  sc_lane: the lane's row (lane & 31)
  // within a 32-row line, its group's 4-byte column (W4A4) and the half swap of sc_col.
  const uint32_t sc_lane = (lane & 31u) * SC_ROW | ((SC_WIN == 8) ? 4u * (lane >> 5) : 0u) | (16u * ((lane >> 2) & 1u));
  auto read_scales = [&](int w, uint32_t (&scw)[4], uint32_t (&sca)[4]) {
    if constexpr (HAS_SC) {
      // lane group g's blocks g*STEPS .. g*STEPS+STEPS-1 as bytes 0.. of one word; the
      // window's column (bits 2-4 of the row offset) enters as one XOR with sc_lane
      const uint8_t* slot = lds + SC_BASE + (uint32_t)((w / CW) & 1) * SLOT;
      const uint32_t off = sc_lane ^ ((uint32_t)(w % CW) * SC_WIN);
      const uint32_t sh = (SC_WIN == 8) ? 0 : 16 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        scw[i] = *reinterpret_cast<const uint32_t*>(slot + (wn * 128 + 32 * i) * SC_ROW + off) >> sh;
      if constexpr (MODE == GEMM_W4A4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          sca[j] = *reinterpret_cast<const uint32_t*>(slot + (BN + wm * 128 + 32 * j) * SC_ROW + off) >> sh;
      }
    }
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nwin = p.nwin;
  uint32_t scw[4] = {0, 0, 0, 0}, sca[4] = {0, 0, 0, 0};
  v4i f0[12], f1[12];
  constexpr int RD = (MODE == GEMM_W4A8) ? 12 : 8;       // ds_read_b128 per fragment set
  constexpr int VM = A_LINES + W_LINES;                  // tile DMA loads per wave per window
  // tile loads issued under step 0 (VM1: weight tile) and at the hand-over (VM0: activation tile)
  constexpr int VM1 = W_LINES, VM0 = A_LINES;
  // loads allowed in flight when the hand-over has to see window w+1 complete
  constexpr int WAIT_VM = (NS - 2) * VM;

  // prologue: window 0 and scale chunk 0 resident, chunk 1 and windows 1 .. NS-1 in flight
  // (the chunk first, so the hand-over wait counts below see only tile loads after it),
  // step-0 fragments and scales read.
  issue_loads(0);
  if constexpr (HAS_SC) issue_chunk(0);
  __builtin_amdgcn_s_waitcnt(0);          // vmcnt/lgkmcnt = 0: stage 0 and chunk 0 written
  __syncthreads();
  if constexpr (HAS_SC)
    if (nchunks > 1) issue_chunk(1);
#pragma unroll
  for (int k = 1; k < NS; ++k)
    if (k < nwin) issue_loads(k);
  read_frags<MODE>(f0, a_at(0), w_at(0), wm, wn, lane, 0);
  read_scales(0, scw, sca);

  // One window.  PEND: the step-0 tile loads go out (the weight tile of window w+NS-1,
  // whose activation tile went out at the previous hand-over).  STEADY: the hand-over
  // waits for window w+1 only and refills the slot this window releases with the
  // activation tile of window w+NS.  The tail waits for everything and loads no tiles.
  // Memory-free MFMAs cannot be sunk past the barrier: every step is its own scheduling
  // region.  sl is window w's ring slot w mod NS, a std::integral_constant where the
  // caller knows it: the slot arithmetic and the LDS read addresses then fold into
  // constants and instruction offsets.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  auto window = [&](int w, auto pend_tag, auto steady_tag, auto sl) {
    constexpr bool PEND = decltype(pend_tag)::value;
    constexpr bool STEADY = decltype(steady_tag)::value;
    const uint32_t s0 = (uint32_t)sl, s1 = (s0 + 1) % NS, sp = (s0 + NS - 1) % NS;
    const uint8_t* la = a_at(s0);
    const uint8_t* lw = w_at(s0);
    if constexpr (HAS_SC)
      if (chunk_due(w)) issue_chunk(w / CW + 1);
    __builtin_amdgcn_sched_barrier(0);
    // step-0 tile loads, spread over the reads of step 0
    auto pend_loads = [&](int k) {
      if constexpr (PEND) {
        if (dma_after(k, VM1, RD) > 0) issue_line(sp, w + NS - 1, I1{}, k * VM1 / RD);
      }
    };
    // Steps 0 .. STEPS-2, one scheduling region each (a region boundary after every step
    // keeps the compiler from mixing steps, which reuses fragment registers early and
    // forces waits on reads just issued): the next step's fragments are read under this
    // step's 16 MFMAs.  Step 0 also carries the pending weight-tile loads, at most one per
    // two MFMAs so that the four waves together stay within the rate the vector memory
    // pipeline accepts (a full queue stalls the wave, and with it the matrix core).  The
    // next window's scales are read a region early: their chunk is resident and visible
    // at least one hand-over before (CW >= 3), so the copy after the hand-over never waits.
    uint32_t scw_n[4], sca_n[4];
    if constexpr (C::STEPS == 4) {
      read_frags<MODE>(f1, la, lw, wm, wn, lane, 1, pend_loads);
      mfma16<MODE, 0>(acc, f0, scw, sca);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // 1 DS read
        if (PEND && dma_after(r, VM1, RD) > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // 1 VMEM
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // 2 MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frags<MODE>(f0, la, lw, wm, wn, lane, 2);
      read_scales(w + 1, scw_n, sca_n);
      mfma16<MODE, 1>(acc, f1, scw, sca);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      read_frags<MODE>(f1, la, lw, wm, wn, lane, 3);
      mfma16<MODE, 2>(acc, f0, scw, sca);
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    } else {
      read_frags<MODE>(f1, la, lw, wm, wn, lane, 1, pend_loads);
      read_scales(w + 1, scw_n, sca_n);
      mfma16<MODE, 0>(acc, f0, scw, sca);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (PEND && r < RD && dma_after(r, VM1, RD) > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    // Hand-over, kept on this side of the last step's MFMAs (which touch no memory and
    // would otherwise be moved below the barrier, exposing the LDS reads).
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (STEADY && WAIT_VM > 0)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(WAIT_VM));   // window w+1 landed
    else
      __builtin_amdgcn_s_waitcnt(0);
    stage_barrier();                      // every wave is past stage `cur`
    __builtin_amdgcn_sched_barrier(0);
    // refill the slot just released, spread over the next window's step-0 reads
    read_frags<MODE>(f0, a_at(s1), w_at(s1), wm, wn, lane, 0, [&](int k) {
      if constexpr (STEADY) {
        if (dma_after(k, VM0, RD) > 0) issue_line(s0, w + NS, I0{}, k * VM0 / RD);
      }
    });
    if constexpr (C::STEPS == 4)
      mfma16<MODE, 3>(acc, f1, scw, sca);
    else
      mfma16<MODE, 1>(acc, f1, scw, sca);
    constexpr int MPR = 16 / RD > 1 ? 2 : 1;   // MFMAs per read slot (16 / RD rounded down, at most 2)
#pragma unroll
    for (int r = 0; r < 16 / MPR; ++r) {
      if (r < RD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);                               // DS read
      if (STEADY && r < RD && dma_after(r, VM0, RD) > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);   // VMEM
      __builtin_amdgcn_sched_group_barrier(0x008, MPR, 1);                                         // MFMA
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      scw[i] = scw_n[i];
      sca[i] = sca_n[i];
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  auto slot_of = [](int w) { return (uint32_t)w % NS; };
  int w = 0;
  if (nwin > NS) {
    window(0, F_{}, T_{}, slot_of(0));
    // steady windows NS at a time, window 1 + NS k + u in the constant slot (1 + u) mod NS
    auto one = [&](auto u_tag) {
      constexpr int U = decltype(u_tag)::value;
      if constexpr (U < NS) window(w + U, T_{}, T_{}, std::integral_constant<uint32_t, (1 + U) % NS>{});
    };
    static_assert(NS <= 3, "one() covers three steady windows per group");
    for (w = 1; w + NS <= nwin - NS; w += NS) {
      one(std::integral_constant<int, 0>{});
      one(std::integral_constant<int, 1>{});
      one(std::integral_constant<int, 2>{});
    }
    for (; w < nwin - NS; ++w) window(w, T_{}, T_{}, slot_of(w));
    window(w, T_{}, F_{}, slot_of(w));
    ++w;
  }
  for (; w < nwin; ++w) window(w, F_{}, F_{}, slot_of(w));

  // ---- epilogue: fp32 -> bf16 (RNE) ----
  if (p.vec16 && n0 + BN <= p.N) {
      // A lane holds 4 consecutive columns of 32 different rows, so a direct store touches
      // 32 cache lines per instruction.  Each wave instead parks 32 rows of its 128 x 128
      // sub-tile at a time in its own 8 KB of the last window's activation slot (free after
      // the last hand-over barrier; 16-byte chunk c of row r at slot c ^ (r & 15), spreading
      // the writes of 16 rows over all banks) and stores 4 whole 256-byte row segments per
      // instruction.
      uint8_t* sub = a_at(slot_of(nwin - 1)) + wave * (32u * 256u);
      const int mw = m0 + (int)wm * 128;
      uint16_t* obase = p.out + (int64_t)mw * p.ld_out + n0 + wn * 128;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            float v0 = acc[i][j][4 * pp + 0], v1 = acc[i][j][4 * pp + 1];
            float v2 = acc[i][j][4 * pp + 2], v3 = acc[i][j][4 * pp + 3];
            if constexpr (MODE == GEMM_W4A8) {
              v0 *= p.a_scale;
              v1 *= p.a_scale;
              v2 *= p.a_scale;
              v3 *= p.a_scale;
            }
            const uint32_t chunk = 4 * i + pp, er = lane & 31;
            *reinterpret_cast<v2u*>(sub + er * 256 + ((chunk ^ (er & 15)) << 4) + 8 * (lane >> 5)) =
                v2u{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
            if (pp == 3) __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t row = 4 * q + (lane >> 4), c = lane & 15;
          const v4i v = *reinterpret_cast<const v4i*>(sub + row * 256 + ((c ^ (row & 15)) << 4));
          const int orow = 32 * j + (int)row;
          if (mw + orow < p.M) {
            v4i* dst = reinterpret_cast<v4i*>(obase + (int64_t)orow * p.ld_out + c * 8);
            if constexpr (STREAM)
              __builtin_nontemporal_store(v, dst);
            else
              *dst = v;
          }
        }
      }
  } else {
    store_partial_tile<MODE>(p, acc, lane, wm, wn, m0, n0);
  }
}

}  // namespace

#if defined(MXQ_GEMM_SCALED_OBJECT)
// The scaled instances, launched from launch_gemm in the main object.
void launch_fast_w4a4(const Params& p, unsigned grid, hipStream_t stream) {
  if (p.stream_out)
    hipLaunchKernelGGL((gemm_fast_kernel<GEMM_W4A4, true>), dim3(grid), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_fast_kernel<GEMM_W4A4, false>), dim3(grid), dim3(NT), 0, stream, p);
}
void launch_fast_w4a8(const Params& p, unsigned grid, hipStream_t stream) {
  if (p.stream_out)
    hipLaunchKernelGGL((gemm_fast_kernel<GEMM_W4A8, true>), dim3(grid), dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL((gemm_fast_kernel<GEMM_W4A8, false>), dim3(grid), dim3(NT), 0, stream, p);
}
#else
// Defined in the scaled-GEMM object (gemm_scaled.hip: this file, built with machine
// sinking off).
void launch_fast_w4a4(const Params& p, unsigned grid, hipStream_t stream);
void launch_fast_w4a8(const Params& p, unsigned grid, hipStream_t stream);

namespace {

// ---------------------------------------------------------------------------------
// W4A4 with the dynamic activation quantization fused in ("AMD Quark adds native W4A8
// mixed-precision for Wan2.2 ...", section "Quark quantization pipeline and mixed-precision
// selection": activations are quantized to MXFP4 dynamically; "AMD Quark: 1.92x faster
// FLUX.1-dev ...", section "MXFP4 quantization for diffusion models": the GEMM takes MXFP4
// with no separate conversion phase).  Unquantized activations enter the GEMM; every
// workgroup quantizes its own activation rows window by window into LDS -- codes in the
// swizzled layout that the W4A4 kernels stage from HBM, scale bytes in a per-window
// plane -- and runs the W4A4 MFMA steps on them in the same order, so each output is
// bit-identical to mx_quantize_kernel followed by the W4A4 GEMM.
//
// The quantization is mx_quantize_kernel's: four lanes own a 32-element block (8 bf16 or
// 4 binary32 ... per lane), the block maximum is an integer max over the sign-cleared
// patterns reduced across the lanes of the block by DPP, the scale byte comes from its
// exponent field, and the codes from the gfx950 scaled FP4 conversion of the exact
// values (the bf16 form converts the same binary32 number the widened f32 form does).

// One lane's 8 bf16 of a 32-element block held by 4 consecutive lanes -> 4 code bytes
// (element 2j in the low nibble of byte j); s = the block's scale byte (equal across the
// quad).  The quad maximum uses DPP operands of v_max_u32 directly; the scale is formed
// as max(s << 23, 2^-127's pattern), the binary32 2^(s-127) for every s including 0.
template <bool UOS>
__device__ __forceinline__ unsigned mx_quant8_bf16(v4i d, unsigned& s) {
  const unsigned d0 = (unsigned)d[0], d1 = (unsigned)d[1], d2 = (unsigned)d[2], d3 = (unsigned)d[3];
  v2h m = __builtin_elementwise_max(__builtin_bit_cast(v2h, d0 & 0x7FFF7FFFu), __builtin_bit_cast(v2h, d1 & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(v2h, d2 & 0x7FFF7FFFu));
  m = __builtin_elementwise_max(m, __builtin_bit_cast(v2h, d3 & 0x7FFF7FFFu));
  unsigned amax = max((unsigned)m[0], (unsigned)m[1]);
  amax = max(amax, (unsigned)__builtin_amdgcn_mov_dpp((int)amax, 0xB1, 0xF, 0xF, true));   // lane ^ 1
  amax = max(amax, (unsigned)__builtin_amdgcn_mov_dpp((int)amax, 0x4E, 0xF, 0xF, true));   // lane ^ 2
  const unsigned e = amax >> 7;
  if constexpr (UOS) {
    s = scale_byte_uos(e, (amax & 0x7Fu) > 0x68u ? 1u : 0u);
  } else {
    const unsigned t = __builtin_elementwise_sub_sat(e, 2u);
    s = e == 255u ? 255u : t;
  }
  const float scale = __uint_as_float(max(s << 23, 0x00400000u));
  // byte 0 first; the other bytes of the first destination are overwritten after
  unsigned r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(d0, __builtin_bit_cast(bf16x2, d0), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, d1), scale, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, d2), scale, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, d3), scale, 3);
  return r;
}

// One lane's 4 binary32 of a 32-element block held by 8 consecutive lanes -> 2 code
// bytes (low 16 bits); s = the block's scale byte.
template <bool UOS>
__device__ __forceinline__ unsigned mx_quant4_f32(v4i d, unsigned& s) {
  unsigned m = max(max((unsigned)d[0] & 0x7FFFFFFFu, (unsigned)d[1] & 0x7FFFFFFFu),
                   max((unsigned)d[2] & 0x7FFFFFFFu, (unsigned)d[3] & 0x7FFFFFFFu));
  m = quad_max_u32(m);
  const unsigned amax = max(m, (unsigned)__shfl_xor((int)m, 4));
  const unsigned e = amax >> 23;
  s = UOS ? scale_byte_uos(e, (amax & 0x7FFFFFu) > 0x680000u ? 1u : 0u) : scale_byte_from_exp(e);
  const float scale = e8m0_to_f32(s);
  unsigned r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __int_as_float(d[0]), __int_as_float(d[1]), scale, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __int_as_float(d[2]), __int_as_float(d[3]), scale, 1);
  return r;
}

// Epilogue of the fused kernel (the fast kernels' epilogue): fp32 -> bf16 (RNE).  Runs
// after the last hand-over barrier; the staged path reuses the first 128 KB of `lds`.
__device__ __forceinline__ void store_tile_w4a4(const Params& p, v16f (&acc)[4][4], uint8_t* lds, uint32_t wave,
                                                uint32_t lane, uint32_t wm, uint32_t wn, int m0, int n0) {
  const uint32_t r32 = lane & 31, g = lane >> 5;
  if (p.vec16 && n0 + BN <= p.N) {
    __syncthreads();
    uint8_t* sub = lds + wave * (128u * 256u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t row = 32 * j + r32;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint32_t chunk = 4 * i + pp;
          *reinterpret_cast<v2u*>(sub + row * 256 + ((chunk ^ (row & 15)) << 4) + 8 * g) =
              v2u{pack_bf16x2(acc[i][j][4 * pp + 0], acc[i][j][4 * pp + 1]),
                  pack_bf16x2(acc[i][j][4 * pp + 2], acc[i][j][4 * pp + 3])};
        }
    }
    const int mw = m0 + (int)wm * 128;
    uint16_t* obase = p.out + (int64_t)mw * p.ld_out + n0 + wn * 128;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      const uint32_t row = 4 * q + (lane >> 4), c = lane & 15;
      const v4i v = *reinterpret_cast<const v4i*>(sub + row * 256 + ((c ^ (row & 15)) << 4));
      if (mw + (int)row < p.M) *reinterpret_cast<v4i*>(obase + (int64_t)row * p.ld_out + c * 8) = v;
    }
    return;
  }
  const bool full = p.vec_store && m0 + BM <= p.M && n0 + BN <= p.N;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + (int)(wm * 128 + 32 * j + r32);
    uint16_t* orow = p.out + (int64_t)min(m, p.M - 1) * p.ld_out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int n = n0 + (int)(wn * 128 + 32 * i + 8 * pp + 4 * g);
        const unsigned lo = pack_bf16x2(acc[i][j][4 * pp + 0], acc[i][j][4 * pp + 1]);
        const unsigned hi = pack_bf16x2(acc[i][j][4 * pp + 2], acc[i][j][4 * pp + 3]);
        if (full) {
          *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
        } else if (m < p.M) {
          if (p.vec_store && n + 4 <= p.N) {
            *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
          } else {
            if (n + 0 < p.N) orow[n + 0] = (uint16_t)lo;
            if (n + 1 < p.N) orow[n + 1] = (uint16_t)(lo >> 16);
            if (n + 2 < p.N) orow[n + 2] = (uint16_t)hi;
            if (n + 3 < p.N) orow[n + 3] = (uint16_t)(hi >> 16);
          }
        }
      }
    }
  }
}

// Tile order of the eight-wave and fused kernels: the fast kernels' XCD-aware raster with
// groups one m-tile wide, so the workgroups an XCD runs at once share one activation panel
// (these kernels stream bf16 activations; measured against 4 m-tiles: bf16 reference
// 7.82 -> 7.72 ms, fused W4A4 4.59 -> 4.28 ms; the four-wave scaled kernels keep GROUP_M,
// where one m-tile is 7 % slower).
__device__ __forceinline__ void tile_origin(const Params& p, int& m0, int& n0) {
  constexpr int GROUP_M = 1;
  const int nt = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int q8 = nt >> 3, r8 = nt & 7;
  const int seq = xcd * q8 + min(xcd, r8) + local;
  const int group = seq / (GROUP_M * p.tiles_n);
  const int first_m = group * GROUP_M;
  const int gm = min(GROUP_M, p.tiles_m - first_m);
  const int in_group = seq - group * GROUP_M * p.tiles_n;
  m0 = (first_m + in_group % gm) * BM;
  n0 = (in_group / gm) * BN;
}

// Generic fused kernel: any K (a multiple of 32), bf16 or binary32 activations, scale
// planes of any alignment.  One LDS stage, register-staged weights; each window is
// quantized in four passes, then its four MFMA steps run (no overlap).
template <bool F32, bool UOS>
__global__ __launch_bounds__(NT, 1) void gemm_w4a4_fused_generic_kernel(Params p) {
  constexpr uint32_t A_TILE = BM * 128, W_TILE = BN * 128;
  constexpr uint32_t AS_OFF = A_TILE + W_TILE;               // activation scale plane: [256 rows][8]
  constexpr uint32_t STAGE = 4 * 128 * 256;                  // the epilogue's staging: 4 waves x 128 rows x 256 bytes
  __shared__ __attribute__((aligned(16))) uint8_t lds[AS_OFF + BM * 8 > STAGE ? AS_OFF + BM * 8 : STAGE];
  constexpr int W_CH = W_TILE / 16 / NT;                     // 8 chunks of 16 bytes per thread
  constexpr int E = F32 ? 4 : 2;                             // bytes per activation element

  const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t wm = wave & 1, wn = wave >> 1;
  int m0, n0;
  tile_origin(p, m0, n0);
  const uint32_t rows_a = (uint32_t)min(BM, p.M - m0), rows_w = (uint32_t)min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.a_row_bytes, rows_a * p.a_row_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w + (int64_t)n0 * p.w_row_bytes, rows_w * p.w_row_bytes);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(p.w_scales + (int64_t)n0 * p.scale_row_bytes, rows_w * p.scale_row_bytes);
  const uint32_t k_bytes = (uint32_t)p.scale_row_bytes * 32u * E;   // K elements in bytes

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const uint32_t w_c = tid % 8, w_r = tid / 8;
  uint32_t sw_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sw_off[i] = (wn * 128 + 32 * i + (lane & 31)) * p.scale_row_bytes;

  for (int w = 0; w < p.nwin; ++w) {
    // weights and their scales into registers
    v4i stw[W_CH];
    const uint32_t wbase = (uint32_t)w * 128 + w_c * 16;
    const bool w_in = wbase + 16 <= p.w_row_bytes;
#pragma unroll
    for (int i = 0; i < W_CH; ++i)
      stw[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_in ? (w_r + i * 32) * p.w_row_bytes + wbase : 0x80000000u, 0, 0);
    uint32_t scw[4], sca[4];
    const uint32_t col = (uint32_t)w * 8 + 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) scw[i] = load_scale4(rsw, sw_off[i], col, p.scale_row_bytes, p.scale_dword_ok);
    __syncthreads();                     // the previous window's MFMAs are done with LDS
#pragma unroll
    for (int i = 0; i < W_CH; ++i) *reinterpret_cast<v4i*>(lds + A_TILE + swz128(w_r + i * 32, w_c)) = stw[i];
    // activations: wave v quantizes rows 64v .. 64v+63, 16 rows per pass
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
      if constexpr (!F32) {
        // a load covers 2 rows x 256 elements; lane l: row +l/32, elements 8 (l%32) ..
        const uint32_t h = lane >> 5, b = (lane & 31) >> 2, k = lane & 3;
        const uint32_t ebyte = (uint32_t)w * 512 + 16 * (lane & 31);
        const bool in = ebyte + 16 <= k_bytes;
        v4i d[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t row = 64 * wave + 16 * q + 2 * i + h;
          d[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, in ? row * p.a_row_bytes + ebyte : 0x80000000u, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t row = 64 * wave + 16 * q + 2 * i + h;
          unsigned s;
          const unsigned c = mx_quant8_bf16<UOS>(d[i], s);
          *reinterpret_cast<unsigned*>(lds + swz128(row, b) + 4 * k) = c;
          if (k == 0) lds[AS_OFF + row * 8 + b] = (uint8_t)s;
        }
      } else {
        // a load covers 1 row x 256 elements; lane l: elements 4l .. 4l+3
        const uint32_t b = lane >> 3, k = lane & 7;
        const uint32_t ebyte = (uint32_t)w * 1024 + 16 * lane;
        const bool in = ebyte + 16 <= k_bytes;
        v4i d[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t row = 64 * wave + 16 * q + i;
          d[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, in ? row * p.a_row_bytes + ebyte : 0x80000000u, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t row = 64 * wave + 16 * q + i;
          unsigned s;
          const unsigned c = mx_quant4_f32<UOS>(d[i], s);
          *reinterpret_cast<uint16_t*>(lds + swz128(row, b) + 2 * k) = (uint16_t)c;
          if (k == 0) lds[AS_OFF + row * 8 + b] = (uint8_t)s;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sca[j] = *reinterpret_cast<const uint32_t*>(lds + AS_OFF + (wm * 128 + 32 * j + (lane & 31)) * 8 + 4 * (lane >> 5));
    mfma_step<GEMM_W4A4, 0>(acc, lds, lds + A_TILE, wm, wn, lane, scw, sca);
    mfma_step<GEMM_W4A4, 1>(acc, lds, lds + A_TILE, wm, wn, lane, scw, sca);
    mfma_step<GEMM_W4A4, 2>(acc, lds, lds + A_TILE, wm, wn, lane, scw, sca);
    mfma_step<GEMM_W4A4, 3>(acc, lds, lds + A_TILE, wm, wn, lane, scw, sca);
  }
  store_tile_w4a4(p, acc, lds, wave, lane, wm, wn, m0, n0);
}

// ---------------------------------------------------------------------------------
// bf16 reference GEMM: 16 x 16 x 32 MFMAs, eight waves (two per SIMD).
//
// Under these GEMMs the chip runs below its top clock to stay within its power, and the
// energy of an MFMA grows with the operand bits that toggle.  With real bf16 operands a
// register-only loop of v_mfma_f32_16x16x32_bf16 sustains ~14 % more than one of
// v_mfma_f32_32x32x16_bf16, at the same work per element.  The 16 x 16 shape needs two
// waves per SIMD to keep the matrix core fed.  Each wave owns 128 (m) x 64 (n): 8
// activation and 4 weight fragments of 16 rows, 32 accumulators of 4 registers, 32 MFMAs
// per step, two steps (K = 32 each) per 64-element window.
//
// Lane layout of the 16 x 16 MFMA (pinned on the GPU): lane l holds row l & 15 of a
// fragment and K-group g = l >> 4 (8 bf16 each); both operands use the same layout, so
// any assignment of K to lane groups that they share is valid.  Lane group g at step t
// reads the 16-byte chunk g + 4t of its rows: with the 128-byte-row swizzle, the four
// lane groups of a ds_read_b128 then touch distinct banks (chunk 2g + t conflicts).  The
// output of block (i, j) sits in lane l as columns 4g .. 4g+3 of row l & 15.
//
// Pipeline (same DMA, swizzle and epilogue staging as gemm_fast_kernel): three activation
// slots and two weight slots of 32 KB.  The hand-over of window w releases both of its
// slots; the weight tile of window w+2, then the activation tile of window w+3, go out
// under the next step's MFMAs, so activation tiles (streamed from HBM) get about two
// windows to land and weight tiles one.  Tile order: groups one m-tile wide
// (tile_origin).  Measured on the Wan2.2 FFN-down shape against the 32 x 32 eight-wave
// kernel it replaces: 7.40-7.64 ms vs 7.53-7.83 ms.
constexpr int NT16 = 512;

// Step-t fragments of one LDS stage: f[0..3] weight rows wn*64 + 16i + (l & 15),
// f[4..11] activation rows wm*128 + 16j + (l & 15); after(k) runs after the k-th read.
template <class After>
__device__ __forceinline__ void read_frags_bf16(v4i (&f)[12], const uint8_t* la, const uint8_t* lw, uint32_t wm,
                                                uint32_t wn, uint32_t lane, int t, After&& after) {
  const uint32_t r16 = lane & 15, chunk = (lane >> 4) + 4 * t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = *reinterpret_cast<const v4i*>(lw + swz128(wn * 64 + 16 * i + r16, chunk));
    after(i);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    f[4 + j] = *reinterpret_cast<const v4i*>(la + swz128(wm * 128 + 16 * j + r16, chunk));
    after(4 + j);
  }
}

__device__ __forceinline__ void mfma_bf16_step(v4f (&acc)[4][8], const v4i (&f)[12]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f[i]),
                                                          __builtin_bit_cast(bf16x8, f[4 + j]), acc[i][j], 0, 0, 0);
}

// Scheduling pattern of one MFMA region: unit I is one fragment read, then (DMA) one tile
// load when the VMN loads spread over the RDN reads fall there, then its share of the
// region's MFMAS MFMAs.
template <int ID, int R, int MFMAS, int VMN, bool DMA, int I>
__device__ __forceinline__ void sched_unit() {
  __builtin_amdgcn_sched_group_barrier(0x100, 1, ID);
  if constexpr (DMA && dma_after(I, VMN, R) > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, ID);
  constexpr int n = (I + 1) * MFMAS / R - I * MFMAS / R;
  if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x008, n, ID);
}
template <int ID, int R, int MFMAS, int VMN, bool DMA, int... Is>
__device__ __forceinline__ void sched_units(std::integer_sequence<int, Is...>) {
  (sched_unit<ID, R, MFMAS, VMN, DMA, Is>(), ...);
}

__global__ __launch_bounds__(NT16, 1) void gemm_bf16_kernel(Params p) {
  constexpr int WAVES = NT16 / 64;
  constexpr int NA = 3, NW = 2;                       // activation / weight ring slots
  constexpr uint32_t RB = 128;                        // bytes per row per window (64 bf16)
  constexpr uint32_t TILE = BM * RB;                  // 32 KB (BM == BN)
  constexpr int LINES = (int)(TILE / 1024 / WAVES);   // 4 DMA lines per wave per tile
  constexpr int ROWS_PER_LINE = 1024 / RB;
  constexpr uint32_t W_BASE = NA * TILE;
  static_assert(BM == BN && 4 * 128 * 256 <= (NA + NW) * TILE, "output staging fits the rings");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(NA + NW) * TILE];

  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const uint32_t wm = wave & 1, wn = wave >> 1;
  int m0, n0;
  tile_origin(p, m0, n0);
  const uint32_t rows_a = (uint32_t)min(BM, p.M - m0), rows_w = (uint32_t)min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.a_row_bytes, rows_a * p.a_row_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w + (int64_t)n0 * p.w_row_bytes, rows_w * p.w_row_bytes);

  // direct-to-LDS lines: LDS line q holds rows 8q .. 8q+7; lane i lands at byte 16 i, in
  // row i / 8 at slot i % 8, and fetches the chunk the swizzle maps there (the swizzle
  // term (r >> 1) & 7 depends on the line's parity)
  const uint32_t drow = lane >> 3, dslot = lane & 7;
  const uint32_t swz_even = (dslot ^ ((drow >> 1) & 7u)) * 16, swz_odd = (dslot ^ (((8u + drow) >> 1) & 7u)) * 16;
  const uint32_t a_voff0 = drow * p.a_row_bytes + swz_even, a_voff1 = drow * p.a_row_bytes + swz_odd;
  const uint32_t w_voff0 = drow * p.w_row_bytes + swz_even, w_voff1 = drow * p.w_row_bytes + swz_odd;
  auto a_slot = [&](int w) { return lds + (uint32_t)(w % NA) * TILE; };
  auto w_slot = [&](int w) { return lds + W_BASE + (uint32_t)(w % NW) * TILE; };
  auto issue_a = [&](int w, int j) {
    const uint32_t line = wave * LINES + j;
    load_line_to_lds(ra, a_slot(w) + line * 1024, (line & 1) ? a_voff1 : a_voff0,
                     (uint32_t)w * RB + line * ROWS_PER_LINE * p.a_row_bytes);
  };
  auto issue_w = [&](int w, int j) {
    const uint32_t line = wave * LINES + j;
    load_line_to_lds(rw, w_slot(w) + line * 1024, (line & 1) ? w_voff1 : w_voff0,
                     (uint32_t)w * RB + line * ROWS_PER_LINE * p.w_row_bytes);
  };

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
  v4i f0[12], f1[12];
  constexpr int RD = 12;                              // ds_read_b128 per fragment set
  constexpr int VM = 2 * LINES;                       // tile loads after each hand-over

  // prologue: window 0 resident; then, in the order the steady state issues them, the
  // activation tile of window 1, the weight tile of window 1, the activation tile of window 2
#pragma unroll
  for (int j = 0; j < LINES; ++j) {
    issue_a(0, j);
    issue_w(0, j);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < LINES; ++j) issue_a(1, j);
#pragma unroll
  for (int j = 0; j < LINES; ++j) issue_w(1, j);
#pragma unroll
  for (int j = 0; j < LINES; ++j) issue_a(2, j);
  read_frags_bf16(f0, a_slot(0), w_slot(0), wm, wn, lane, 0, [](int) {});

  // One window: step 0 on f0 under the reads of step 1 into f1; the hand-over waits for
  // window w+1 (only the activation tile of window w+2 may still be in flight) and
  // releases window w's slots; step 1 on f1 under the reads of window w+1's step 0 into
  // f0 and the DMA of the weight tile of window w+2 and the activation tile of window
  // w+3.  Every window refills, the last ones with tiles past K: buffer loads that stay
  // inside each resource (bytes of later rows, or zeros past its end) into slots no later
  // window reads.  A single loop body keeps the register allocator from splitting the
  // 32 accumulators between loop copies.
  const int nwin = p.nwin;
  for (int w = 0; w < nwin; ++w) {
    read_frags_bf16(f1, a_slot(w), w_slot(w), wm, wn, lane, 1, [](int) {});
    mfma_bf16_step(acc, f0);
    sched_units<0, RD, 32, 0, false>(std::make_integer_sequence<int, RD>{});
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(LINES));   // window w+1 landed
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags_bf16(f0, a_slot(w + 1), w_slot(w + 1), wm, wn, lane, 0, [&](int k) {
      if (dma_after(k, VM, RD) > 0) {
        const int j = k * VM / RD;
        if (j < LINES)
          issue_w(w + NW, j);
        else
          issue_a(w + NA, j - LINES);
      }
    });
    mfma_bf16_step(acc, f1);
    sched_units<1, RD, 32, VM, true>(std::make_integer_sequence<int, RD>{});
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: fp32 -> bf16 (RNE); lane l holds columns 4g .. 4g+3 of row l & 15 of
  // every 16 x 16 block ----
  const uint32_t r16 = lane & 15, g = lane >> 4;
  if (p.vec16 && n0 + BN <= p.N) {
    // park the wave's 128 (m) x 64 (n) sub-tile in LDS (16-byte chunk c of row r at
    // c ^ (r & 7)) and store whole 128-byte row segments; the loop's last loads are waited
    // for by the barrier's release fence before any wave overwrites the rings
    __syncthreads();
    uint8_t* sub = lds + wave * (128u * 128u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t row = 16 * j + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4f& v = acc[i][j];
        const uint32_t chunk = 2 * i + (g >> 1);
        *reinterpret_cast<v2u*>(sub + row * 128 + ((chunk ^ (row & 7)) << 4) + 8 * (g & 1)) =
            v2u{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
    const int mw = m0 + (int)wm * 128;
    uint16_t* obase = p.out + (int64_t)mw * p.ld_out + n0 + wn * 64;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t row = 8 * q + (lane >> 3), c = lane & 7;
      const v4i v = *reinterpret_cast<const v4i*>(sub + row * 128 + ((c ^ (row & 7)) << 4));
      if (mw + (int)row < p.M) *reinterpret_cast<v4i*>(obase + (int64_t)row * p.ld_out + c * 8) = v;
    }
    return;
  }
  // partial column tiles: a lane owns 4 consecutive columns per store
  const bool full = p.vec_store && m0 + BM <= p.M && n0 + BN <= p.N;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + (int)(wm * 128 + 16 * j + r16);
    uint16_t* orow = p.out + (int64_t)min(m, p.M - 1) * p.ld_out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + (int)(wn * 64 + 16 * i + 4 * g);
      const v4f& v = acc[i][j];
      const unsigned lo = pack_bf16x2(v[0], v[1]), hi = pack_bf16x2(v[2], v[3]);
      if (full) {
        *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
      } else if (m < p.M) {
        if (p.vec_store && n + 4 <= p.N) {
          *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
        } else {
          if (n + 0 < p.N) orow[n + 0] = (uint16_t)lo;
          if (n + 1 < p.N) orow[n + 1] = (uint16_t)(lo >> 16);
          if (n + 2 < p.N) orow[n + 2] = (uint16_t)hi;
          if (n + 3 < p.N) orow[n + 3] = (uint16_t)(hi >> 16);
        }
      }
    }
  }
}

// Four blocks' worth of one lane's activations -> codes, with the block maxima reduced
// across the quad by a transpose: the lanes of a quad hold 8 elements of each of four
// blocks (their chunks i = 0..3); two DPP exchanges leave lane k with block k's maximum,
// so each lane forms one scale (its own block's byte, returned in s) and broadcasts it
// back to the quad for the conversion.  codes[i] = 4 code bytes of chunk i.
template <bool UOS>
__device__ __forceinline__ int mx_quad4_scale_bf16(const v4i (&d)[4], uint32_t lane, unsigned& s) {
  unsigned m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned x0 = (unsigned)d[i][0], x1 = (unsigned)d[i][1], x2 = (unsigned)d[i][2], x3 = (unsigned)d[i][3];
    v2h mm = __builtin_elementwise_max(__builtin_bit_cast(v2h, x0 & 0x7FFF7FFFu), __builtin_bit_cast(v2h, x1 & 0x7FFF7FFFu));
    mm = __builtin_elementwise_max(mm, __builtin_bit_cast(v2h, x2 & 0x7FFF7FFFu));
    mm = __builtin_elementwise_max(mm, __builtin_bit_cast(v2h, x3 & 0x7FFF7FFFu));
    m[i] = max((unsigned)mm[0], (unsigned)mm[1]);
  }
  const bool hi_pair = (lane & 2) != 0, odd = (lane & 1) != 0;
  // exchange with lane ^ 2: keep blocks {2p, 2p+1} (p = lane bit 1), send the other pair
  const unsigned snd0 = hi_pair ? m[0] : m[2], snd1 = hi_pair ? m[1] : m[3];
  const unsigned kp0 = hi_pair ? m[2] : m[0], kp1 = hi_pair ? m[3] : m[1];
  const unsigned t0 = max(kp0, (unsigned)__builtin_amdgcn_mov_dpp((int)snd0, 0x4E, 0xF, 0xF, true));
  const unsigned t1 = max(kp1, (unsigned)__builtin_amdgcn_mov_dpp((int)snd1, 0x4E, 0xF, 0xF, true));
  // exchange with lane ^ 1: keep block 2p + (lane bit 0)
  const unsigned snd = odd ? t0 : t1, kp = odd ? t1 : t0;
  const unsigned amax = max(kp, (unsigned)__builtin_amdgcn_mov_dpp((int)snd, 0xB1, 0xF, 0xF, true));
  const unsigned e = amax >> 7;
  if constexpr (UOS) {
    s = scale_byte_uos(e, (amax & 0x7Fu) > 0x68u ? 1u : 0u);
  } else {
    const unsigned t = __builtin_elementwise_sub_sat(e, 2u);
    s = e == 255u ? 255u : t;
  }
  return (int)max(s << 23, 0x00400000u);
}

// The conversion half of the above: scale_bits = this lane's block scale (binary32 bits).
__device__ __forceinline__ void mx_quad4_convert_bf16(const v4i (&d)[4], int scale_bits, unsigned (&codes)[4]) {
  auto convert = [&](auto i_tag) {
    constexpr int I = decltype(i_tag)::value;
    // block I's scale lives in lane I of the quad: quad_perm [I, I, I, I]
    const float sc = __int_as_float(__builtin_amdgcn_mov_dpp(scale_bits, I * 0x55, 0xF, 0xF, true));
    const unsigned x0 = (unsigned)d[I][0], x1 = (unsigned)d[I][1], x2 = (unsigned)d[I][2], x3 = (unsigned)d[I][3];
    unsigned r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(x0, __builtin_bit_cast(bf16x2, x0), sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x1), sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x2), sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, x3), sc, 3);
    codes[I] = r;
  };
  convert(std::integral_constant<int, 0>{});
  convert(std::integral_constant<int, 1>{});
  convert(std::integral_constant<int, 2>{});
  convert(std::integral_constant<int, 3>{});
}

// Fast fused kernel (bf16 activations; K a whole number of 256-element windows; weight
// scale rows and planes on 16-byte boundaries), eight waves (two per SIMD).  Each wave
// owns a 64 (m) x 128 (n) sub-tile: 4 weight x 2 activation fragments of 32x32x64 MFMAs,
// 8 accumulators; every 32 x 32 output block gets the same MFMAs in the same order as in
// gemm_fast_kernel<GEMM_W4A4>, hence the same bits.  Weight tiles stream through a
// two-slot ring with 32-byte weight scale chunks; the activation tile is quantized in the
// kernel.
// Activation window w+1 is quantized during window w, a quarter per MFMA step: wave v
// quantizes rows 32v + 8q .. +7 of quarter q from registers loaded D steps earlier (1 KB =
// 2 rows x 256 elements per load instruction, 4 per quarter), and writes 4 code bytes per
// chunk into the two-slot code ring (the swizzled layout the W4A4 kernels stage) and its
// block's scale byte into a two-slot [256 x 8] plane.  Quarter 0 of window w+1 is
// quantized after the hand-over barrier of window w-1, which releases its slot; quarters
// 1-3 under steps 0-2 of window w.  A step runs as two units in source order, fenced
// from each other: 4 MFMAs, 3 fragment reads and half of the quantization each.
constexpr int NT8 = 512;

template <bool UOS, int D>
__global__ __launch_bounds__(NT8, 1) void gemm_w4a4_fused8_kernel(Params p) {
  static_assert(D == 1 || D == 2 || D == 4, "load lead of 1, 2 or 4 steps");
  constexpr int WAVES = NT8 / 64;
  constexpr uint32_t A_TILE = BM * 128, W_TILE = BN * 128;   // code tiles, 32 KB each
  constexpr int W_LINES = (int)(W_TILE / 1024 / WAVES);       // 4 weight lines per wave per window
  constexpr uint32_t W_BASE = 2 * A_TILE;
  constexpr uint32_t SC_ROW = 32;                             // weight scale chunk: 32 bytes per row
  constexpr int CW = 4;                                       // windows per chunk
  constexpr uint32_t SLOT = BN * SC_ROW;
  constexpr int SC_LINES = (int)(SLOT / 1024 / WAVES);        // 1
  constexpr uint32_t SC_BASE = W_BASE + 2 * W_TILE;
  constexpr uint32_t AS_BASE = SC_BASE + 2 * SLOT;
  constexpr uint32_t AS_SLOT = BM * 8;                        // [256 rows][8] scale bytes
  __shared__ __attribute__((aligned(1024))) uint8_t lds[AS_BASE + 2 * AS_SLOT];
  static_assert(AS_BASE + 2 * AS_SLOT >= 8u * 16384u, "epilogue staging fits");

  const uint32_t tid = threadIdx.x, lane = tid & 63;
  const uint32_t wave = (uint32_t)__builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const uint32_t wm = wave & 3, wn = wave >> 2;
  int m0, n0;
  tile_origin(p, m0, n0);
  const uint32_t rows_a = (uint32_t)min(BM, p.M - m0), rows_w = (uint32_t)min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a + (int64_t)m0 * p.a_row_bytes, rows_a * p.a_row_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w + (int64_t)n0 * p.w_row_bytes, rows_w * p.w_row_bytes);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(p.w_scales + (int64_t)n0 * p.scale_row_bytes, rows_w * p.scale_row_bytes);
  const uint32_t pitch = p.a_row_bytes;

  const uint32_t wr = lane >> 3, wsl = lane & 7;
  const uint32_t w_voff0 = wr * p.w_row_bytes + ((wsl ^ ((wr >> 1) & 7u)) * 16);
  const uint32_t w_voff1 = wr * p.w_row_bytes + ((wsl ^ (((8u + wr) >> 1) & 7u)) * 16);
  const uint32_t sc_voff = (lane >> 1) * p.scale_row_bytes + (((lane & 1) ^ ((lane >> 3) & 1)) * 16);
  // load i of quarter q covers rows 32v + 8q + 2i + (lane / 32), elements 8 (lane % 32) ..
  // of the window; the code slot of row r, block b is b ^ ((r >> 1) & 7) = b ^ (4 (q & 1) + i)
  const uint32_t h = lane >> 5, b = (lane & 31) >> 2, k = lane & 3;
  const uint32_t a_voff = h * pitch + 16 * (lane & 31);
  const uint32_t cw0 = wave * 4096u + h * 128u + 4u * k + (b << 4);
  const uint32_t sw0 = (wave * 32u + 2u * k + h) * 8u + b;     // scale byte of the quad's block k

  auto issue_w_line = [&](int w, int par, int j) {
    const uint32_t line = wave * W_LINES + j;
    load_line_to_lds(rw, lds + W_BASE + (uint32_t)par * W_TILE + line * 1024, (line & 1) ? w_voff1 : w_voff0,
                     (uint32_t)w * 128 + line * 8 * p.w_row_bytes);
  };
  const int nwin = p.nwin;
  const int nchunks = (nwin + CW - 1) / CW;
  auto issue_chunk = [&](int c) {
    uint8_t* slot = lds + SC_BASE + (uint32_t)(c & 1) * SLOT;
#pragma unroll
    for (int j = 0; j < SC_LINES; ++j) {
      const uint32_t line = wave * SC_LINES + j;
      load_line_to_lds(rsw, slot + line * 1024, sc_voff, (uint32_t)c * SC_ROW + line * 32 * p.scale_row_bytes);
    }
  };
  auto chunk_due = [&](int w) { return w >= CW && w % CW == 0 && w / CW + 1 < nchunks; };
  auto read_w_scale = [&](int w, uint32_t ln, int i) {
    const uint8_t* slot = lds + SC_BASE + (uint32_t)((w / CW) & 1) * SLOT;
    const uint32_t col = sc_col((uint32_t)(w % CW) * 8 + 4 * (ln >> 5), ln & 31);
    return *reinterpret_cast<const uint32_t*>(slot + (wn * 128 + 32 * i + (ln & 31)) * SC_ROW + col);
  };
  auto read_a_scale = [&](int par, uint32_t ln, int j) {
    return *reinterpret_cast<const uint32_t*>(lds + AS_BASE + (uint32_t)par * AS_SLOT +
                                              (wm * 64 + 32 * j + (ln & 31)) * 8 + 4 * (ln >> 5));
  };
  // fragment kk (0-3: weight rows wn*128 + 32kk, 4-5: activation rows wm*64 + 32(kk-4)) of
  // MFMA step t from slot `par`
  auto read_frag = [&](int par, uint32_t ln, int t, int kk) {
    const uint32_t chunk = (ln >> 5) * 4 + t;
    const uint8_t* base = kk < 4 ? lds + W_BASE + (uint32_t)par * W_TILE : lds + (uint32_t)par * A_TILE;
    const uint32_t row = kk < 4 ? wn * 128 + 32 * kk + (ln & 31) : wm * 64 + 32 * (kk - 4) + (ln & 31);
    return *reinterpret_cast<const v4i*>(base + swz128(row, chunk));
  };
  auto load_act = [&](int v, int q, int i) {
    return __builtin_amdgcn_raw_buffer_load_b128(ra, a_voff, (uint32_t)(32 * wave + 8 * q + 2 * i) * pitch + (uint32_t)v * 512u,
                                                 0);
  };
  // quantize quarter q (4 loads) into code / scale slot `par`: the block scales (and the
  // scale bytes), then the codes
  auto quant_scale = [&](int par, int q, const v4i (&d)[4]) {
    unsigned s;
    const int bits = mx_quad4_scale_bf16<UOS>(d, lane, s);
    lds[AS_BASE + (uint32_t)par * AS_SLOT + q * 64 + sw0] = (uint8_t)s;
    return bits;
  };
  auto quant_codes = [&](int par, int q, const v4i (&d)[4], int bits) {
    unsigned c[4];
    mx_quad4_convert_bf16(d, bits, c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<unsigned*>(lds + (uint32_t)par * A_TILE + q * 1024 + 256 * i +
                                   (cw0 ^ ((uint32_t)(4 * (q & 1) + i) << 4))) = c[i];
  };
  auto quant_quarter = [&](int par, int q, const v4i (&d)[4]) { quant_codes(par, q, d, quant_scale(par, q, d)); };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // prologue: weight window 0 and chunk 0 in flight; activation window 0 and quarter 0 of
  // window 1 quantized one quarter at a time; then chunk 1, the first D quarters of the
  // steady-state lead and weight window 1 in flight, in the order the steady state keeps
  // them (loads past the last window read zeros or unused bytes, and nothing reads what
  // they deliver); step-0 fragments and scales read.
#pragma unroll
  for (int j = 0; j < W_LINES; ++j) issue_w_line(0, 0, j);
  issue_chunk(0);
#pragma unroll
  for (int Q = 0; Q < 5; ++Q) {
    v4i d[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = load_act(Q / 4, Q % 4, i);
    if (Q / 4 < nwin) quant_quarter((Q / 4) & 1, Q % 4, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  issue_chunk(1);
  v4i stg[D][4];
#pragma unroll
  for (int Q = 5; Q < 5 + D; ++Q)
#pragma unroll
    for (int i = 0; i < 4; ++i) stg[(Q % 4) % D][i] = load_act(Q / 4, Q % 4, i);
#pragma unroll
  for (int j = 0; j < W_LINES; ++j) issue_w_line(1, 1, j);
  uint32_t scw[4], sca[2];
  v4i f0[6], f1[6];
#pragma unroll
  for (int kk = 0; kk < 6; ++kk) f0[kk] = read_frag(0, lane, 0, kk);
#pragma unroll
  for (int i = 0; i < 4; ++i) scw[i] = read_w_scale(0, lane, i);
#pragma unroll
  for (int j = 0; j < 2; ++j) sca[j] = read_a_scale(0, lane, j);

  // One window w with slot parity PAR = w & 1 (a constant in the steady state).  Region r
  // (the MFMAs of step r) quantizes global quarter 4w + r + 5 (window w+1 quarters 1..3,
  // then window w+2 quarter 0) from the registers loaded D regions earlier and loads
  // quarter 4w + r + 5 + D into them.  TAIL windows check each against the window count
  // and drain all loads at the hand-over.
  auto window = [&](int w, int PAR, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    uint32_t ln = lane;
    asm volatile("" : "+v"(ln));
    if (chunk_due(w)) issue_chunk(w / CW + 1);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t scw_n[4], sca_n[2];
    auto region = [&](auto r_tag, v4i (&fc)[6], v4i (&fn)[6]) {
      constexpr int R = decltype(r_tag)::value;
      constexpr int QC = (R + 1) & 3, VC = (R + 5) >> 2;           // quarter quantized: window w + VC
      constexpr int QL = (R + 1 + D) & 3, VL = (R + 5 + D) >> 2;   // quarter loaded: window w + VL
      constexpr int IX = QC % D;
      static_assert(QL % D == IX, "ring slot");
      const int PC = (PAR + VC) & 1;                               // code / scale slot quantized into
      const bool q_ok = !TAIL || w + VC < nwin;
      const bool l_ok = !TAIL || w + VL < nwin;
      int bits = 0;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int i = 2 * u; i < 2 * u + 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(fc[i]), widen(fc[4 + j]), acc[i][j], 4, 4,
                                                                        R, (int)scw[i], R, (int)sca[j]);
#pragma unroll
        for (int kk = 3 * u; kk < 3 * u + 3; ++kk) {
          if constexpr (R < 3) {
            fn[kk] = read_frag(PAR, ln, R + 1, kk);
          } else {
            fn[kk] = read_frag(PAR ^ 1, ln, 0, kk);
            if (kk < W_LINES && (!TAIL || w + 2 < nwin)) issue_w_line(w + 2, PAR, kk);
          }
        }
        if constexpr (R == 1) {
          scw_n[2 * u] = read_w_scale(w + 1, ln, 2 * u);
          scw_n[2 * u + 1] = read_w_scale(w + 1, ln, 2 * u + 1);
        }
        if constexpr (R == 3) {
          if (u == 1 && (!TAIL || w + 2 < nwin)) issue_w_line(w + 2, PAR, 3);
          sca_n[u] = read_a_scale(PAR ^ 1, ln, u);
        }
        // unit 0: block scales of the quarter; unit 1: its codes, then (after a fence, so
        // that they reuse the registers just read) the loads of the next quarter
        if (u == 0) {
          if (q_ok) bits = quant_scale(PC, QC, stg[IX]);
        } else {
          if (q_ok) quant_codes(PC, QC, stg[IX], bits);
          __builtin_amdgcn_sched_barrier(0);
          if (l_ok) {
#pragma unroll
            for (int i = 0; i < 4; ++i) stg[IX][i] = load_act(w + VL, QL, i);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    region(std::integral_constant<int, 0>{}, f0, f1);
    region(std::integral_constant<int, 1>{}, f1, f0);
    region(std::integral_constant<int, 2>{}, f0, f1);
    // hand-over: weight window w+1 landed (at least 16 loads went out after it), this
    // wave's code and scale writes for window w+1 done; then every wave is past its reads
    // of window w's slots
    if constexpr (TAIL)
      __builtin_amdgcn_s_waitcnt(0);
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * (D < 3 ? D : 3)));
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    region(std::integral_constant<int, 3>{}, f1, f0);
#pragma unroll
    for (int i = 0; i < 4; ++i) scw[i] = scw_n[i];
#pragma unroll
    for (int j = 0; j < 2; ++j) sca[j] = sca_n[j];
  };
  constexpr int TAIL_WINDOWS = D <= 2 ? 2 : 3;
  const int steady = nwin - TAIL_WINDOWS;
  int w = 0;
  for (; w + 1 < steady; w += 2) {
    window(w, 0, std::false_type{});
    window(w + 1, 1, std::false_type{});
  }
  if (w < steady) {
    window(w, 0, std::false_type{});
    ++w;
  }
  for (; w < nwin; ++w) window(w, w & 1, std::true_type{});

  // ---- epilogue: fp32 -> bf16 (RNE), staged per wave through 16 KB of LDS ----
  const uint32_t r32 = lane & 31, g = lane >> 5;
  if (p.vec16 && n0 + BN <= p.N) {
    __syncthreads();
    uint8_t* sub = lds + wave * (64u * 256u);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t row = 32 * j + r32;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const uint32_t chunk = 4 * i + pp;
          *reinterpret_cast<v2u*>(sub + row * 256 + ((chunk ^ (row & 15)) << 4) + 8 * g) =
              v2u{pack_bf16x2(acc[i][j][4 * pp + 0], acc[i][j][4 * pp + 1]),
                  pack_bf16x2(acc[i][j][4 * pp + 2], acc[i][j][4 * pp + 3])};
        }
    }
    const int mw = m0 + (int)wm * 64;
    uint16_t* obase = p.out + (int64_t)mw * p.ld_out + n0 + wn * 128;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t row = 4 * q + (lane >> 4), c = lane & 15;
      const v4i v = *reinterpret_cast<const v4i*>(sub + row * 256 + ((c ^ (row & 15)) << 4));
      if (mw + (int)row < p.M) *reinterpret_cast<v4i*>(obase + (int64_t)row * p.ld_out + c * 8) = v;
    }
    return;
  }
  const bool full = p.vec_store && m0 + BM <= p.M && n0 + BN <= p.N;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + (int)(wm * 64 + 32 * j + r32);
    uint16_t* orow = p.out + (int64_t)min(m, p.M - 1) * p.ld_out;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        const int n = n0 + (int)(wn * 128 + 32 * i + 8 * pp + 4 * g);
        const unsigned lo = pack_bf16x2(acc[i][j][4 * pp + 0], acc[i][j][4 * pp + 1]);
        const unsigned hi = pack_bf16x2(acc[i][j][4 * pp + 2], acc[i][j][4 * pp + 3]);
        if (full) {
          *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
        } else if (m < p.M) {
          if (p.vec_store && n + 4 <= p.N) {
            *reinterpret_cast<v2u*>(orow + n) = v2u{lo, hi};
          } else {
            if (n + 0 < p.N) orow[n + 0] = (uint16_t)lo;
            if (n + 1 < p.N) orow[n + 1] = (uint16_t)(lo >> 16);
            if (n + 2 < p.N) orow[n + 2] = (uint16_t)hi;
            if (n + 3 < p.N) orow[n + 3] = (uint16_t)(hi >> 16);
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(GemmMode mode, const void* a, const uint8_t* a_scales, const void* w,
                       const uint8_t* w_scales, float a_scale, int64_t M, int64_t N, int64_t K,
                       uint16_t* out, int64_t ld_out, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  Params p;
  p.a = static_cast<const uint8_t*>(a);
  p.a_scales = a_scales;
  p.w = static_cast<const uint8_t*>(w);
  p.w_scales = w_scales;
  p.out = out;
  p.ld_out = ld_out;
  p.M = (int)M;
  p.N = (int)N;
  p.scale_row_bytes = (uint32_t)(K / 32);
  auto aligned_to = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) % a) == 0; };
  p.scale_dword_ok = ((K / 32) % 4 == 0 && aligned_to(a_scales, 4) && aligned_to(w_scales, 4)) ? 1 : 0;
  p.a_scale = a_scale;
  p.vec_store = (ld_out % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0) ? 1 : 0;
  p.vec16 = (ld_out % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) ? 1 : 0;
  // Short K loops write more output per tile of input: marking those output stores
  // non-temporal keeps the operand panels that neighbouring tiles re-read in L2 (measured:
  // 2-4.5 % faster for K = 3072-6144, within about 1 % either way at K = 8192-13824).
  p.stream_out = K <= kStreamOutMaxK ? 1 : 0;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(NT);
  // the fast path needs whole windows and, with scales, scale rows and planes on 16-byte
  // boundaries (they are fetched 16 bytes per lane)
  const bool scales_ok = (K / 32) % 16 == 0 && aligned_to(a_scales, 16) && aligned_to(w_scales, 16);
  auto launch = [&](auto mode_tag, uint32_t a_row_bytes, uint32_t w_row_bytes, bool needs_scales) {
    constexpr int MD = decltype(mode_tag)::value;
    p.a_row_bytes = a_row_bytes;
    p.w_row_bytes = w_row_bytes;
    if (K > 0 && K % Fast<MD>::K_WIN == 0 && (scales_ok || !needs_scales)) {
      p.nwin = (int)(K / Fast<MD>::K_WIN);
      // the bf16 reference runs its 16 x 16 eight-wave kernel; the scaled modes the
      // four-wave 32 x 32 kernel, whose W4A4 MFMA order the fused kernel reproduces bit
      // for bit (eight waves of 32 x 32 MFMAs measured slower for both scaled modes)
      if constexpr (MD == GEMM_BF16) {
        hipLaunchKernelGGL(gemm_bf16_kernel, grid, dim3(NT16), 0, stream, p);
      } else if constexpr (MD == GEMM_W4A4) {
        launch_fast_w4a4(p, grid.x, stream);
      } else {
        launch_fast_w4a8(p, grid.x, stream);
      }
    } else {
      p.nwin = (int)((K + Cfg<MD>::K_WIN - 1) / Cfg<MD>::K_WIN);
      hipLaunchKernelGGL(gemm_generic_kernel<MD>, grid, block, 0, stream, p);
    }
  };
  switch (mode) {
    case GEMM_W4A4:
      launch(std::integral_constant<int, GEMM_W4A4>{}, (uint32_t)(K / 2), (uint32_t)(K / 2), true);
      break;
    case GEMM_W4A8:
      launch(std::integral_constant<int, GEMM_W4A8>{}, (uint32_t)K, (uint32_t)(K / 2), true);
      break;
    case GEMM_BF16:
      launch(std::integral_constant<int, GEMM_BF16>{}, (uint32_t)(K * 2), (uint32_t)(K * 2), false);
      break;
  }
  return hipGetLastError();
}


hipError_t launch_gemm_w4a4_fused(const void* a, bool f32, int64_t ld_a, const uint8_t* w, const uint8_t* w_scales,
                                  int64_t M, int64_t N, int64_t K, bool uos, uint16_t* out, int64_t ld_out,
                                  hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  Params p;
  p.a = static_cast<const uint8_t*>(a);
  p.a_scales = nullptr;
  p.w = w;
  p.w_scales = w_scales;
  p.out = out;
  p.ld_out = ld_out;
  p.M = (int)M;
  p.N = (int)N;
  p.a_row_bytes = (uint32_t)(ld_a * (f32 ? 4 : 2));
  p.w_row_bytes = (uint32_t)(K / 2);
  p.scale_row_bytes = (uint32_t)(K / 32);
  auto aligned_to = [](const void* q, uintptr_t al) { return (reinterpret_cast<uintptr_t>(q) % al) == 0; };
  p.scale_dword_ok = ((K / 32) % 4 == 0 && aligned_to(w_scales, 4)) ? 1 : 0;
  p.a_scale = 1.0f;
  p.vec_store = (ld_out % 4 == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0) ? 1 : 0;
  p.vec16 = (ld_out % 8 == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) ? 1 : 0;
  p.stream_out = 0;
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(NT);
  const bool fast = !f32 && K > 0 && K % 256 == 0 && (K / 32) % 16 == 0 && aligned_to(w_scales, 16);
  if (fast) {
    p.nwin = (int)(K / 256);
    if (uos)
      hipLaunchKernelGGL((gemm_w4a4_fused8_kernel<true, 2>), grid, dim3(NT8), 0, stream, p);
    else
      hipLaunchKernelGGL((gemm_w4a4_fused8_kernel<false, 2>), grid, dim3(NT8), 0, stream, p);
  } else {
    p.nwin = (int)((K + 255) / 256);
    if (f32) {
      if (uos)
        hipLaunchKernelGGL((gemm_w4a4_fused_generic_kernel<true, true>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((gemm_w4a4_fused_generic_kernel<true, false>), grid, block, 0, stream, p);
    } else {
      if (uos)
        hipLaunchKernelGGL((gemm_w4a4_fused_generic_kernel<false, true>), grid, block, 0, stream, p);
      else
        hipLaunchKernelGGL((gemm_w4a4_fused_generic_kernel<false, false>), grid, block, 0, stream, p);
    }
  }
  return hipGetLastError();
}

#endif  // MXQ_GEMM_SCALED_OBJECT

}  // namespace mxq
