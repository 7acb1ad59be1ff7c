// kda_device.h -- device-side helpers shared by the HIP kernels of this library
// (gfx950 / CDNA4 only): element types, MFMA tile products, small utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kChunk = 64;   // tokens per chunk of the chunkwise schedule
constexpr int kThreads = 256;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR lanes, every lane receiving its group's
// sum, in registers: DPP quad permutes for lane distance 1 and 2, the half-row
// and row mirrors for 4 and 8 (once the smaller groups hold equal sums a
// mirror reads the other half), and the row swap of gfx950 for 16.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR >= 1 && LPR <= 32, "group of at most 32 lanes");
  if constexpr (LPR >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (LPR >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (LPR >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (LPR >= 32) {
    // rows 2i and 2i+1 trade places between the two results
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// e^x = 2^(x log2 e) on the hardware exponential (v_exp_f32).  Rounding
// x log2 e costs a relative error of about |x| 2^-24 on top of the
// instruction's own; -inf gives exactly 0.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// A gate from its logarithm.
__device__ __forceinline__ float gate_from_log(float g) { return fast_exp(g); }

// A gate from a softplus logit: exp(-softplus(g)) = 1 / (1 + e^g), on the
// hardware reciprocal; large g gives 0, very negative g gives 1.
__device__ __forceinline__ float gate_from_softplus_logit(float g) { return __builtin_amdgcn_rcpf(1.f + fast_exp(g)); }

__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + fast_exp(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// 1 / max(|x|, 1e-12) from a sum of squares (the normalisation of a vector).
__device__ __forceinline__ float inv_norm(float sumsq) { return __builtin_amdgcn_rsqf(fmaxf(sumsq, 1e-24f)); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <typename E> __device__ __forceinline__ float to_f(E x) { return (float)x; }
template <typename E> __device__ __forceinline__ E from_f(float x) { return (E)x; }

// ---------------------------------------------------------------------------
// 16x16 output tiles on the matrix cores.  Lane l of a wave holds, for a tile
// product D = A (16 x K) * B (K x 16):
//   A operand: row l%16, k-slots g*KPL .. g*KPL+KPL-1 with g = l/16
//   B operand: column l%16, the same k-slots
//   D result : rows 4*g + r (r = 0..3), column l%16
// The k-slot order only has to agree between A and B.
// ---------------------------------------------------------------------------
template <typename E, int KS> struct Mma;

template <> struct Mma<bf16, 32> {      // v_mfma_f32_16x16x32_bf16
  static constexpr int KS = 32, KPL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const bf16 *p) {
    return *reinterpret_cast<const frag *>(p);
  }
};

template <> struct Mma<bf16, 16> {      // v_mfma_f32_16x16x16_bf16
  static constexpr int KS = 16, KPL = 4;
  typedef bf16x4 frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const bf16 *p) {
    return *reinterpret_cast<const frag *>(p);
  }
};

template <int KSunused> struct MmaF32 {  // v_mfma_f32_16x16x4_f32
  static constexpr int KS = 4, KPL = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float *p) { return *p; }
};
template <> struct Mma<float, 32> : MmaF32<32> {};
template <> struct Mma<float, 16> : MmaF32<16> {};

// The widest product that divides K.
template <typename E, int K> struct MmaFor {
  typedef Mma<E, (K % 32 == 0) ? 32 : 16> type;
};

// acc += A_rows(16 x K) * Bt_rows(16 x K)^T, where a_row / bt_row point at the
// first element of this lane's A row and B column (B stored transposed, i.e.
// one row of Bt per output column).  K must be a multiple of M::KS.
template <typename M, int K, typename E>
__device__ __forceinline__ f32x4 mma_rows(const E *a_row, const E *bt_row, f32x4 acc) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += M::KS)
    acc = M::mma(M::load(a_row + k0 + g * M::KPL), M::load(bt_row + k0 + g * M::KPL), acc);
  return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// One output of a causal convolution of width four: taps w[0..3] on the
// values of tokens t-3 .. t, summed in that order (one product, then three
// fused multiply-adds; every caller that must agree bit for bit uses this).
__device__ __forceinline__ float conv_taps(const f32x4 &w, float x0, float x1, float x2, float x3) {
  float y = w[0] * x0;
  y = __builtin_fmaf(w[1], x1, y);
  y = __builtin_fmaf(w[2], x2, y);
  return __builtin_fmaf(w[3], x3, y);
}

}  // namespace kda
