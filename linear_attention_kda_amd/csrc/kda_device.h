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

// A gate from its logarithm: e^g = 2^(g log2 e) on the hardware exponential
// (v_exp_f32).  Rounding g log2 e costs a relative error of about |g| 2^-24
// on top of the instruction's own; g = -inf gives exactly 0.
__device__ __forceinline__ float gate_from_log(float g) {
  return __builtin_amdgcn_exp2f(g * 1.4426950408889634f);
}

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

}  // namespace kda
