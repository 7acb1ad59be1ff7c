// kda_decode.hip -- single-token KDA step (decode) for gfx950.
//
// Method: page "Kimi Delta Attention (KDA)" (brain.bigb.es), opening update
// equation, taken token by token (the "fused recurrent" schedule of section
// "Two schedules for one recurrence").  Value rows of the state are
// independent, so each row r of S (d_v x d_k) is streamed through registers
// once:
//     s~ = S[r,:] * alpha           (forget: key channels are the columns)
//     vhat_r = s~ . k ;  e_r = beta (v_r - vhat_r)
//     S[r,:] = s~ + e_r k
//     o_r = scale * S[r,:] . q = scale * (s~ . q + e_r (k . q))
//
// The state is HBM-resident fp32 and dominates the traffic (one read and one
// write per step), so the kernel is laid out for bandwidth: a lane owns 16
// contiguous channels of one row (four 16-byte loads), LPR = d_k/16 lanes
// cover a row, and the two dot products are reduced across those lanes with
// cross-lane swizzles.  One workgroup per (sequence, head).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

struct DecodeKArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  float *S;
  void *o;
  float scale;
};

template <typename E>
__device__ __forceinline__ void load16(const E *p, float *out);

template <>
__device__ __forceinline__ void load16<bf16>(const bf16 *p, float *out) {
  const bf16x8 a = *reinterpret_cast<const bf16x8 *>(p);
  const bf16x8 b = *reinterpret_cast<const bf16x8 *>(p + 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[i] = (float)a[i];
    out[8 + i] = (float)b[i];
  }
}

template <>
__device__ __forceinline__ void load16<float>(const float *p, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 x = reinterpret_cast<const f32x4 *>(p)[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * i + j] = x[j];
  }
}

template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

template <int DK, int DV, typename E>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeKArgs a) {
  constexpr int LPR = DK / 16;        // lanes per state row
  constexpr int RPW = 64 / LPR;       // rows per wave per pass
  constexpr int RPB = 4 * RPW;        // rows per workgroup per pass
  constexpr int PASSES = (DV + RPB - 1) / RPB;

  const size_t u = blockIdx.x;        // (sequence, head) unit
  const int w = wave_id(), l = lane_id();
  const int sub = l % LPR, rloc = l / LPR;
  const int c0 = 16 * sub;

  float kk[16], qq[16], al[16];
  load16<E>(reinterpret_cast<const E *>(a.k) + u * DK + c0, kk);
  load16<E>(reinterpret_cast<const E *>(a.q) + u * DK + c0, qq);
  load16<float>(a.alpha + u * DK + c0, al);
  float kq = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) kq += kk[i] * qq[i];
  kq = group_sum<LPR>(kq);
  const float beta = a.beta[u];
  const E *vrow = reinterpret_cast<const E *>(a.v) + u * DV;
  E *orow = reinterpret_cast<E *>(a.o) + u * DV;
  float *S = a.S + u * DV * DK;

  f32x4 s[PASSES][4];
  // issue every load of this lane's rows first
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = p * RPB + w * RPW + rloc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[p][i] = r < DV ? reinterpret_cast<const f32x4 *>(S + (size_t)r * DK + c0)[i] : zero4();
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = p * RPB + w * RPW + rloc;
    // rows past DV only occur for tiny d_v with wide rows; their lanes idle
    float st[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) st[4 * i + j] = s[p][i][j] * al[4 * i + j];
    float d1 = 0.f, d2 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      d1 += st[i] * kk[i];
      d2 += st[i] * qq[i];
    }
    d1 = group_sum<LPR>(d1);
    d2 = group_sum<LPR>(d2);
    if (r < DV) {
      const float e = beta * ((float)vrow[r] - d1);
      f32x4 outv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) outv[i][j] = st[4 * i + j] + e * kk[4 * i + j];
#pragma unroll
      for (int i = 0; i < 4; ++i) reinterpret_cast<f32x4 *>(S + (size_t)r * DK + c0)[i] = outv[i];
      if (sub == 0) orow[r] = (E)(a.scale * (d2 + e * kq));
    }
  }
}

template <int DK, typename E>
hipError_t run_decode_dv(const DecodeArgs &a, const DecodeKArgs &ka, hipStream_t s) {
  const dim3 grid((unsigned)((size_t)a.N * a.H));
  switch (a.dv) {
    case 16: hipLaunchKernelGGL((decode_kernel<DK, 16, E>), grid, dim3(kThreads), 0, s, ka); break;
    case 32: hipLaunchKernelGGL((decode_kernel<DK, 32, E>), grid, dim3(kThreads), 0, s, ka); break;
    case 64: hipLaunchKernelGGL((decode_kernel<DK, 64, E>), grid, dim3(kThreads), 0, s, ka); break;
    case 128: hipLaunchKernelGGL((decode_kernel<DK, 128, E>), grid, dim3(kThreads), 0, s, ka); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename E>
hipError_t run_decode(const DecodeArgs &a, hipStream_t s) {
  DecodeKArgs ka{a.q, a.k, a.v, a.alpha, a.beta, a.S, a.o, a.scale};
  switch (a.dk) {
    case 16: return run_decode_dv<16, E>(a, ka, s);
    case 32: return run_decode_dv<32, E>(a, ka, s);
    case 64: return run_decode_dv<64, E>(a, ka, s);
    case 128: return run_decode_dv<128, E>(a, ka, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if ((size_t)a.N * a.H == 0) return hipSuccess;
  return a.bf16 ? run_decode<bf16>(a, stream) : run_decode<float>(a, stream);
}

}  // namespace kda
