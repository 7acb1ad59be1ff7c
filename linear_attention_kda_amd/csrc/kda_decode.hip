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
// write per step), so the kernel is laid out for bandwidth: every wave-wide
// state access is one contiguous KiB (lane l takes bytes 16l..16l+15), a lane
// owns 4 channels of one row, LPR = d_k/4 lanes cover a row, and the two dot
// products are summed across those lanes with cross-lane swizzles.  State
// loads and stores carry the nontemporal hint: each state byte is touched
// once per step, and keeping it out of the caches measured faster.  One
// workgroup per (sequence, head).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

struct DecodeKArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  int gate;  // kGateChannel: alpha [N, H, d_k]; kGateScalar: alpha [N, H]; kGateNone: unused
  float *S;
  void *o;
  float scale;
  size_t units;  // sequences x heads
};

template <typename E>
__device__ __forceinline__ void load4(const E *p, float *out);

template <>
__device__ __forceinline__ void load4<bf16>(const bf16 *p, float *out) {
  const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = (float)a[i];
}

template <>
__device__ __forceinline__ void load4<float>(const float *p, float *out) {
  const f32x4 x = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = x[i];
}

template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Work split: a unit's state is NACC wave-wide KiB accesses.  A workgroup of
// four waves takes APW = min(NACC, 8) of them (two per wave), so a d = 128
// unit spreads over 8 workgroups; fewer accesses in flight per wave and more
// workgroups measured closer to the copy bandwidth of the part.
template <int DK, int DV> struct DecodeShape {
  static constexpr int NACC = DV * DK / 256;
  static constexpr int APW = NACC < 8 ? NACC : 8;
  static constexpr int SPLIT = NACC / APW;        // workgroups per unit
  static constexpr int NI = (APW + 3) / 4;        // accesses per wave
};

template <int DK, int DV, typename E>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeKArgs a) {
  typedef DecodeShape<DK, DV> SH;
  constexpr int LPR = DK / 4;                 // lanes per state row
  constexpr int RPA = 64 / LPR;               // rows per wave-wide KiB access
  constexpr int NI = SH::NI;                  // accesses per wave

  // the SPLIT workgroups of a unit get ids congruent mod 8, which the
  // dispatcher sends to one XCD, so k, q and alpha leave HBM once per unit
  const size_t bid = blockIdx.x, slot = bid >> 3;
  const size_t u = (slot / SH::SPLIT) * 8 + (bid & 7);   // (sequence, head) unit
  const int part = (int)(slot % SH::SPLIT);              // which APW KiB of the unit
  if (u >= a.units) return;
  const int w = wave_id(), l = lane_id();
  const int sub = l % LPR, rsub = l / LPR;
  const int c0 = 4 * sub;

  float kk[4], qq[4], al[4];
  load4<E>(reinterpret_cast<const E *>(a.k) + u * DK + c0, kk);
  load4<E>(reinterpret_cast<const E *>(a.q) + u * DK + c0, qq);
  if (a.gate == kGateChannel) {
    load4<float>(a.alpha + u * DK + c0, al);
  } else {
    const float x = a.gate == kGateScalar ? a.alpha[u] : 1.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) al[j] = x;
  }
  const float beta = a.beta[u];
  const E *vrow = reinterpret_cast<const E *>(a.v) + u * DV;
  E *orow = reinterpret_cast<E *>(a.o) + u * DV;
  float *S = a.S + u * DV * DK;

  // issue every state load of this lane first (waves past the workgroup's
  // share only exist when a unit is smaller than four KiB; they skip)
  f32x4 s[NI];
  float vv[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int acc = part * SH::APW + w * NI + i;
    const int r = acc * RPA + rsub;
    if (w * NI + i < SH::APW) {
      s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(S + (size_t)r * DK + c0));
      vv[i] = (float)vrow[r];
    } else {
      s[i] = zero4();
      vv[i] = 0.f;
    }
  }
  float kq = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) kq += kk[j] * qq[j];
  kq = group_sum<LPR>(kq);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int acc = part * SH::APW + w * NI + i;
    const int r = acc * RPA + rsub;
    float st[4], d1 = 0.f, d2 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      st[j] = s[i][j] * al[j];
      d1 += st[j] * kk[j];
      d2 += st[j] * qq[j];
    }
    d1 = group_sum<LPR>(d1);
    d2 = group_sum<LPR>(d2);
    if (w * NI + i < SH::APW) {
      const float e = beta * (vv[i] - d1);
      f32x4 outv;
#pragma unroll
      for (int j = 0; j < 4; ++j) outv[j] = st[j] + e * kk[j];
      __builtin_nontemporal_store(outv, reinterpret_cast<f32x4 *>(S + (size_t)r * DK + c0));
      if (sub == 0) orow[r] = (E)(a.scale * (d2 + e * kq));
    }
  }
}

template <int DK, typename E>
hipError_t run_decode_dv(const DecodeArgs &a, const DecodeKArgs &ka, hipStream_t s) {
  const size_t units = (size_t)a.N * a.H;
  if ((units + 7) / 8 * 8 * DecodeShape<DK, 128>::SPLIT > 0x7fffffffull) return hipErrorInvalidConfiguration;
#define KDA_DECODE_LAUNCH(DV) \
  hipLaunchKernelGGL((decode_kernel<DK, DV, E>), dim3((unsigned)((units + 7) / 8 * 8 * DecodeShape<DK, DV>::SPLIT)), \
                     dim3(kThreads), 0, s, ka)
  switch (a.dv) {
    case 16: KDA_DECODE_LAUNCH(16); break;
    case 32: KDA_DECODE_LAUNCH(32); break;
    case 64: KDA_DECODE_LAUNCH(64); break;
    case 128: KDA_DECODE_LAUNCH(128); break;
    default: return hipErrorInvalidValue;
  }
#undef KDA_DECODE_LAUNCH
  return hipGetLastError();
}

template <typename E>
hipError_t run_decode(const DecodeArgs &a, hipStream_t s) {
  DecodeKArgs ka{a.q, a.k, a.v, a.alpha, a.beta, a.gate, a.S, a.o, a.scale, (size_t)a.N * a.H};
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
