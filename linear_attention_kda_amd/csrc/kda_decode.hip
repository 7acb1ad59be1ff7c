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
// write per launch), so the kernel is laid out for bandwidth: every wave-wide
// state access is one contiguous KiB (lane l takes bytes 16l..16l+15), a lane
// owns 4 channels of one row, LPR = d_k/4 lanes cover a row, and the two dot
// products are summed across those lanes with cross-lane swizzles.  State
// loads and stores carry the nontemporal hint: each state byte is touched
// once per launch, and keeping it out of the caches measured faster.
//
// One launch may carry Tk tokens of each sequence (checking the tokens a
// draft model proposed: page "K3 架构图解", chapter 10, the section on
// speculative decoding):
// the state rows stay in registers across the tokens and the result may go
// to a second buffer, so the state before the launch survives for rollback.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

struct DecodeKArgs {
  const void *q, *k, *v;
  // alpha: [.., H, d_k] for the per-channel forms, [.., H] for the
  // per-token forms, unused without a gate; the log forms hold log(alpha)
  // (the kernel is instantiated per form)
  const float *alpha, *beta;
  const float *S_in;
  float *S_out;  // may be S_in
  void *o;
  float scale;
  unsigned act;    // kAct* input activations
  unsigned units;  // sequences x heads (< 2^31)
  int H, Tk;     // heads; tokens per sequence (inputs are [N, Tk, H, .])
  // CONV instantiations: convolution taps [H, d, kConvTaps] of q, k, v and
  // the convolution state [units, 3, 2 d_k + d_v] (the three raw tokens
  // before the launch's first, q | k | v; read only here)
  const float *conv_q, *conv_k, *conv_v;
  const void *conv_state;
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

// Work split: a unit's state is NACC wave-wide KiB accesses.  A workgroup of
// four waves takes APW = min(NACC, MAXAPW) of them.  With one token per launch
// MAXAPW = 8 (two per wave), so a d = 128 unit spreads over 8 workgroups;
// fewer accesses in flight per wave and more workgroups measured closer to the
// copy bandwidth of the part.
template <int DK, int DV, int MAXAPW = 8> struct DecodeShape {
  static constexpr int NACC = DV * DK / 256;
  static constexpr int APW = NACC < MAXAPW ? NACC : MAXAPW;
  static constexpr int SPLIT = NACC / APW;        // workgroups per unit
  static constexpr int NI = (APW + 3) / 4;        // accesses per wave
};

// Inputs of one token as this lane needs them: 4 channels of k, q, alpha
// and the values of its state rows.
template <int NI> struct TokIn {
  float kk[4], qq[4], al[4], beta, vv[NI];
};

// Marks every value of x as used here: the loads that fill it must have
// completed at this point.
template <int NI>
__device__ __forceinline__ void consume(const TokIn<NI> &x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) asm volatile("" ::"v"(x.kk[j]), "v"(x.qq[j]), "v"(x.al[j]));
#pragma unroll
  for (int i = 0; i < NI; ++i) asm volatile("" ::"v"(x.vv[i]));
  asm volatile("" ::"v"(x.beta));
}

// Several tokens per launch are bound by vector issue, not by the state
// traffic: each token's own work per lane (its loads and conversions, the k.q
// sum, the decayed gates) is shared by the lane's rows, so the multi-token
// kernel gives each workgroup 32 KiB of state (eight rows per lane, two
// workgroups per d = 128 unit).  Four-token launches on 256 x 32 units took
// 265 us with 8 KiB per workgroup, 229 with 16, 221-227 with 32 and 272 with
// 64 (occupancy two waves per SIMD).
constexpr int kMultiAPW = 32;
// With the convolution each lane also holds the taps of its rows and a window
// of four tokens per input: two rows per lane (8 KiB per workgroup) keep that
// in registers.
template <int DK, int DV, int G, bool CONV = false>
using DecodeShapeG = DecodeShape<DK, DV, (G == 1 || CONV) ? 8 : kMultiAPW>;

// CONV: q, k and v go through the short causal convolution (the token and the
// three before it, the first three from the convolution state) before
// anything else, each result rounded to E as the prefill rounds it.
template <int DK, int DV, typename E, int GATE, int G, bool CONV = false>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeKArgs a) {
  typedef DecodeShapeG<DK, DV, G, CONV> SH;
  static_assert(!CONV || G > 1, "the convolution runs in the multi-token kernel");
  constexpr int LPR = DK / 4;                 // lanes per state row
  constexpr int RPA = 64 / LPR;               // rows per wave-wide KiB access
  constexpr int NI = SH::NI;                  // accesses per wave
  constexpr bool FULL = SH::APW % 4 == 0;     // every wave owns NI accesses

  // the SPLIT workgroups of a unit get ids congruent mod 8, which the
  // dispatcher sends to one XCD, so k, q and alpha leave HBM once per unit
  const unsigned bid = blockIdx.x, slot = bid >> 3;
  const unsigned u = (slot / SH::SPLIT) * 8 + (bid & 7);   // (sequence, head) unit
  const int part = (int)(slot % SH::SPLIT);                // which APW KiB of the unit
  if (u >= a.units) return;
  const int w = wave_id(), l = lane_id();
  // RSC: the several-token kernel at d_k = 128 with eight state rows per
  // lane.  Its per-token work is dominated by the two row sums of each row
  // (k.s~ and q.s~, 16 values per lane), so instead of summing each of them
  // over the row's 32 lanes it reduces all 16 together in a reduce-scatter:
  // at each of the five exchange steps a lane keeps half of its values and
  // adds its partner's copy of them, so after 8 + 4 + 2 + 1 + 1 adds a lane
  // holds one complete sum.  For the halves kept to be fixed registers (no
  // per-lane selects at every step), lanes hold their rows in a
  // lane-dependent order and half of them take the q sum in the slots where
  // the others take the k sum: slot i of lane bits b0..b3 holds row (i ^ m),
  // m = 4 (b1^b2) + 2 (b2^b3) + b3, and lanes with b0^b2 set swap the two
  // sums.  With the step partners l^1, l^2, l^7, l^15, l^16 (quad permutes,
  // half-row and row mirrors, row swap) each partner then holds the same row
  // in the slot sent, and every sum is added up in the order group_sum uses.
  // The row's error term e is formed where its k sum landed and spread back
  // to the 32 lanes in three steps (1 + 2 + 4 moves); the lane with the q sum
  // writes the row's output.  The state is read and written in row order (each
  // wave-wide access one contiguous KiB: reading the rows in slot order, 64
  // bytes per row per access, measured 30 % slower) and put into slot order
  // and back through LDS (three conditional swap stages in registers, 96
  // selects each way, measured 1.5 % slower).
  constexpr bool RSC = G > 1 && !CONV && DK == 128 && NI == 8 && FULL;
  const int sub = l % LPR, rsub = l / LPR;
  const int c0 = 4 * sub;
  const int b0 = sub & 1, b1 = (sub >> 1) & 1, b2 = (sub >> 2) & 1, b3 = (sub >> 3) & 1, b4 = (sub >> 4) & 1;
  const int rperm = RSC ? 4 * (b1 ^ b2) + 2 * (b2 ^ b3) + b3 : 0;  // m above
  const bool qkind = RSC && (b0 ^ b2) != 0;                         // slots 0..7 take the q sum
  const int Tk = G == 1 ? 1 : a.Tk;  // >= 1; the G = 1 kernel is launched for one token
  // token t of this unit in the [N, Tk, H, .] inputs (with one token per
  // launch that is the unit itself)
  auto tok_index = [&](int t) -> size_t {
    if constexpr (G == 1) return u;
    const unsigned n = u / (unsigned)a.H, h = u % (unsigned)a.H;
    return ((size_t)n * Tk + t) * a.H + h;
  };

  // rows of this lane; when a unit is smaller than four KiB the waves past
  // its share read a valid row, compute on zeros and store nothing (loads
  // stay unconditional: a branch around a load costs a full wait)
  int rows[NI];
  bool valid[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int acc = w * NI + i;
    valid[i] = FULL || acc < SH::APW;
    rows[i] = (part * SH::APW + (valid[i] ? acc : 0)) * RPA + rsub;
  }

  // RSC: the row in slot 0 (its value entry and its output)
  const int row0 = RSC ? (part * SH::APW + w * NI + rperm) * RPA + rsub : rows[0];
  // RSC: slot i <- row (i ^ rperm) of the lane's rows, and back (the same
  // permutation), through a lane-private strip of LDS: written in one order,
  // read in the other (slot-major, so each access is conflict-free)
  __shared__ f32x4 perm_lds[RSC ? kThreads / 64 : 1][RSC ? NI : 1][64];
  auto slot_order = [&](f32x4 *st) {
    if constexpr (RSC) {
#pragma unroll
      for (int i = 0; i < NI; ++i) perm_lds[w][i][l] = st[i];
#pragma unroll
      for (int i = 0; i < NI; ++i) st[i] = perm_lds[w][i ^ rperm][l];
    }
  };

  // CONV: the taps of this lane's channels and rows, and where a token's raw
  // inputs are (t >= 0: the launch's inputs; t in -3..-1: the state)
  constexpr int CW = 2 * DK + DV;  // elements per token of the convolution state
  f32x4 wk[4], wq[4], wv[NI];
  if constexpr (CONV) {
    const int h = (int)(u % (unsigned)a.H);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      wk[j] = *reinterpret_cast<const f32x4 *>(a.conv_k + ((size_t)h * DK + c0 + j) * kConvTaps);
      wq[j] = *reinterpret_cast<const f32x4 *>(a.conv_q + ((size_t)h * DK + c0 + j) * kConvTaps);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      wv[i] = *reinterpret_cast<const f32x4 *>(a.conv_v + ((size_t)h * DV + rows[i]) * kConvTaps);
  }
  const E *cstate = CONV ? reinterpret_cast<const E *>(a.conv_state) + (size_t)u * 3 * CW : nullptr;
  auto raw_k = [&](int t) {
    return t >= 0 ? reinterpret_cast<const E *>(a.k) + tok_index(t) * DK : cstate + (size_t)(3 + t) * CW + DK;
  };
  auto raw_q = [&](int t) {
    return t >= 0 ? reinterpret_cast<const E *>(a.q) + tok_index(t) * DK : cstate + (size_t)(3 + t) * CW;
  };
  auto raw_v = [&](int t) {
    return t >= 0 ? reinterpret_cast<const E *>(a.v) + tok_index(t) * DV : cstate + (size_t)(3 + t) * CW + 2 * DK;
  };

  // the inputs of G tokens are requested together, so a group costs one
  // memory latency; indexes past the last token re-read the last token
  constexpr int NV = RSC ? 1 : NI;  // value entries a lane reads per token
  TokIn<NV> x[G];
  auto load_group = [&](int t0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int t = min(t0 + g, Tk - 1);
      const size_t ix = tok_index(t);
      if constexpr (CONV) {
        float xk[kConvTaps][4], xq[kConvTaps][4], xv[kConvTaps][NI];
#pragma unroll
        for (int i = 0; i < kConvTaps; ++i) {
          const int tt = t - (kConvTaps - 1) + i;
          load4<E>(raw_k(tt) + c0, xk[i]);
          load4<E>(raw_q(tt) + c0, xq[i]);
          const E *vr = raw_v(tt);
#pragma unroll
          for (int r = 0; r < NI; ++r) xv[i][r] = (float)vr[rows[r]];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[g].kk[j] = (float)(E)conv_taps(wk[j], xk[0][j], xk[1][j], xk[2][j], xk[3][j]);
          x[g].qq[j] = (float)(E)conv_taps(wq[j], xq[0][j], xq[1][j], xq[2][j], xq[3][j]);
        }
#pragma unroll
        for (int r = 0; r < NI; ++r) x[g].vv[r] = (float)(E)conv_taps(wv[r], xv[0][r], xv[1][r], xv[2][r], xv[3][r]);
      } else {
        load4<E>(reinterpret_cast<const E *>(a.k) + ix * DK + c0, x[g].kk);
        load4<E>(reinterpret_cast<const E *>(a.q) + ix * DK + c0, x[g].qq);
      }
      if constexpr (gate_per_channel(GATE)) {
        load4<float>(a.alpha + ix * DK + c0, x[g].al);
      } else {
        const float al = gate_per_token(GATE) ? a.alpha[ix] : 1.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[g].al[j] = al;
      }
      x[g].beta = a.beta[ix];
      if constexpr (!CONV) {
        const E *vrow = reinterpret_cast<const E *>(a.v) + ix * DV;
#pragma unroll
        for (int i = 0; i < NV; ++i) x[g].vv[i] = (float)vrow[RSC ? row0 : rows[i]];
      }
    }
  };
  // this lane's state rows stay in registers across the tokens: one read and
  // one write of the state per launch
  const float *Sin = a.S_in + (size_t)u * DV * DK;
  f32x4 s[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
    s[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(Sin + (size_t)rows[i] * DK + c0));
  if constexpr (!FULL) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (!valid[i]) s[i] = zero4();
  }
  // the state requests leave first: they come from HBM, the token inputs
  // mostly from L2 (measured 1% faster than letting the scheduler pick)
  __builtin_amdgcn_sched_barrier(0);

  // one call site for the group loads: with two (before the loop and at its
  // end) the compiler merges them into the loop header behind a full wait
  for (int t0 = 0; t0 < Tk; t0 += G) {
    load_group(t0);
    if constexpr (RSC)
      if (t0 == 0) slot_order(s);  // after the first inputs are requested
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int t = t0 + g;
      if (G > 1 && t >= Tk) break;
      TokIn<NV> &y = x[g];
      if constexpr (gate_is_log(GATE)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) y.al[j] = gate_from_log(y.al[j]);
      } else if constexpr (gate_is_softplus(GATE)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) y.al[j] = gate_from_softplus_logit(y.al[j]);
      }
      if (a.act & kActQK) {  // q, k <- SiLU, then unit length over d_k (LPR lanes)
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y.kk[j] = silu_f(y.kk[j]);
          y.qq[j] = silu_f(y.qq[j]);
          sk += y.kk[j] * y.kk[j];
          sq += y.qq[j] * y.qq[j];
        }
        const float rk = inv_norm(group_sum<LPR>(sk)), rq = inv_norm(group_sum<LPR>(sq));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          y.kk[j] *= rk;
          y.qq[j] *= rq;
        }
      }
      if (a.act & kActBeta) y.beta = sigmoid_f(y.beta);
      E *orow = reinterpret_cast<E *>(a.o) + tok_index(t) * DV;
      float kq = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) kq += y.kk[j] * y.qq[j];
      kq = group_sum<LPR>(kq);
      // s~ . k = s . (alpha k) and s~ . q = s . (alpha q) (each lane's four
      // channels in order, then summed over the row's lanes), and the update
      // s <- (alpha s) + e k with e k fused into the add: the same arithmetic
      // in every variant, so several tokens per launch equal as many single
      // steps bit for bit, and a gate of one equals no gate
      float ak[4], aq[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ak[j] = y.al[j] * y.kk[j];
        aq[j] = y.al[j] * y.qq[j];
      }
      if constexpr (RSC) {
        // this lane's slot sums (xs) and the ones it hands to its first
        // partner (xo)
        float ps[4], po[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ps[j] = qkind ? aq[j] : ak[j];
          po[j] = qkind ? ak[j] : aq[j];
        }
        float xs[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float xa = s[i][0] * ps[0], xo = s[i][0] * po[0];
#pragma unroll
          for (int j = 1; j < 4; ++j) {
            xa = fmaf(s[i][j], ps[j], xa);
            xo = fmaf(s[i][j], po[j], xo);
          }
          xs[i] = xa + dpp<0xB1>(xo);  // l ^ 1
        }
        float y2[4], y3[2];
#pragma unroll
        for (int i = 0; i < 4; ++i) y2[i] = xs[i] + dpp<0x4E>(xs[i + 4]);   // l ^ 2
#pragma unroll
        for (int i = 0; i < 2; ++i) y3[i] = y2[i] + dpp<0x141>(y2[i + 2]);  // l ^ 7
        const float y4 = y3[0] + dpp<0x140>(y3[1]);                        // l ^ 15
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(y4), __float_as_uint(y4), false, false);
        const float tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // l ^ 16
        // tot: the k sum (or the q sum) of row row0; its e from the k lane
        const float eown = y.beta * (y.vv[0] - tot);
        const float epart = dpp<0xB1>(eown);
        float ee[8];
        ee[0] = qkind ? epart : eown;
        if (qkind && b4 == 0) orow[row0] = (E)(a.scale * (tot + ee[0] * kq));
        ee[1] = dpp<0x140>(ee[0]);
        ee[2] = dpp<0x141>(ee[0]);
        ee[3] = dpp<0x141>(ee[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) ee[i + 4] = dpp<0x4E>(ee[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) s[i][j] = fmaf(ee[i], y.kk[j], s[i][j] * y.al[j]);
      } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          float d1 = s[i][0] * ak[0], d2 = s[i][0] * aq[0];
#pragma unroll
          for (int j = 1; j < 4; ++j) {
            d1 = fmaf(s[i][j], ak[j], d1);
            d2 = fmaf(s[i][j], aq[j], d2);
          }
          d1 = group_sum<LPR>(d1);
          d2 = group_sum<LPR>(d2);
          const float e = y.beta * (y.vv[i] - d1);
#pragma unroll
          for (int j = 0; j < 4; ++j) s[i][j] = fmaf(e, y.kk[j], s[i][j] * y.al[j]);
          if (valid[i] && sub == 0) orow[rows[i]] = (E)(a.scale * (d2 + e * kq));
        }
      }
    }
    // the inputs of a partial last group past Tk are never read; without
    // this the compiler assumes their loads may still be in flight on the
    // back edge and makes the next group's loads wait for every load
    if constexpr (G > 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) consume(x[g]);
    }
  }

  if constexpr (RSC) slot_order(s);
  // the store addresses are formed here rather than held in registers
  // through the token loop (row i of a lane is its first row + i RPA)
  int r0 = (part * SH::APW + w * NI) * RPA + rsub;
  asm volatile("" : "+v"(r0));
  float *sb = a.S_out + (size_t)u * DV * DK + (size_t)r0 * DK + c0;
#pragma unroll
  for (int i = 0; i < NI; ++i)
    if (valid[i]) __builtin_nontemporal_store(s[i], reinterpret_cast<f32x4 *>(sb + (size_t)(i * RPA) * DK));
}

// The convolution state after a launch: the last three raw tokens of (the
// three before the launch, then its Tk tokens), per (sequence, head).  A
// thread owns one channel of a unit and reads its three old values before
// writing, so the update is in place.
template <typename E>
__global__ __launch_bounds__(256) void conv_state_advance_kernel(const E *q, const E *k, const E *v, E *cs, int H,
                                                                 int dk, int dv, int Tk, unsigned units) {
  const unsigned u = blockIdx.x;
  if (u >= units) return;
  const int W = 2 * dk + dv;
  const size_t n = u / (unsigned)H, h = u % (unsigned)H;
  E *st = cs + (size_t)u * 3 * W;
  for (int c = threadIdx.x; c < W; c += blockDim.x) {
    E old[3];
#pragma unroll
    for (int s = 0; s < 3; ++s) old[s] = st[(size_t)s * W + c];
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      const int wi = Tk + s;  // position in (old 0..2, then the Tk tokens)
      E x;
      if (wi < 3) {
        x = old[wi];
      } else {
        const size_t th = (n * Tk + (wi - 3)) * H + h;
        x = c < dk ? q[th * dk + c] : (c < 2 * dk ? k[th * dk + c - dk] : v[th * dv + c - 2 * dk]);
      }
      st[(size_t)s * W + c] = x;
    }
  }
}

// tokens whose inputs are requested together: two measured faster than four
// (with eight rows per lane: 125 VGPRs and four waves per SIMD against 171
// and two; 221-227 against 263 us per four-token launch on the decode
// workload)
constexpr int kTokGroup = 2;

template <int DK, typename E, int GATE>
hipError_t run_decode_dv(const DecodeArgs &a, const DecodeKArgs &ka, hipStream_t s) {
  const size_t units = (size_t)a.N * a.H;
  if ((units + 7) / 8 * 8 * DecodeShape<DK, 128>::SPLIT > 0x7fffffffull) return hipErrorInvalidConfiguration;
#define KDA_DECODE_LAUNCH(DV)                                                                          \
  {                                                                                                    \
    if (a.conv_q) {                                                                                    \
      const dim3 grid((unsigned)((units + 7) / 8 * 8 * DecodeShapeG<DK, DV, kTokGroup, true>::SPLIT)); \
      hipLaunchKernelGGL((decode_kernel<DK, DV, E, GATE, kTokGroup, true>), grid, dim3(kThreads), 0, s,  \
                         ka);                                                                          \
    } else if (a.Tk == 1) {                                                                            \
      const dim3 grid((unsigned)((units + 7) / 8 * 8 * DecodeShapeG<DK, DV, 1>::SPLIT));               \
      hipLaunchKernelGGL((decode_kernel<DK, DV, E, GATE, 1>), grid, dim3(kThreads), 0, s, ka);          \
    } else {                                                                                           \
      const dim3 grid((unsigned)((units + 7) / 8 * 8 * DecodeShapeG<DK, DV, kTokGroup>::SPLIT));       \
      hipLaunchKernelGGL((decode_kernel<DK, DV, E, GATE, kTokGroup>), grid, dim3(kThreads), 0, s, ka);  \
    }                                                                                                  \
  }
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

template <int DK, typename E>
hipError_t run_decode_gate(const DecodeArgs &a, const DecodeKArgs &ka, hipStream_t s) {
  switch (a.gate) {
    case kGateChannel: return run_decode_dv<DK, E, kGateChannel>(a, ka, s);
    case kGateScalar: return run_decode_dv<DK, E, kGateScalar>(a, ka, s);
    case kGateNone: return run_decode_dv<DK, E, kGateNone>(a, ka, s);
    case kGateLogChannel: return run_decode_dv<DK, E, kGateLogChannel>(a, ka, s);
    case kGateLogScalar: return run_decode_dv<DK, E, kGateLogScalar>(a, ka, s);
    case kGateSoftplusChannel: return run_decode_dv<DK, E, kGateSoftplusChannel>(a, ka, s);
    case kGateSoftplusScalar: return run_decode_dv<DK, E, kGateSoftplusScalar>(a, ka, s);
  }
  return hipErrorInvalidValue;
}

template <typename E>
hipError_t run_decode(const DecodeArgs &a, hipStream_t s) {
  DecodeKArgs ka{a.q, a.k, a.v, a.alpha, a.beta, a.S_in, a.S, a.o, a.scale, a.act, (unsigned)((size_t)a.N * a.H),
                 a.H, a.Tk, a.conv_q, a.conv_k, a.conv_v, a.conv_state};
  hipError_t e = hipErrorInvalidValue;
  switch (a.dk) {
    case 16: e = run_decode_gate<16, E>(a, ka, s); break;
    case 32: e = run_decode_gate<32, E>(a, ka, s); break;
    case 64: e = run_decode_gate<64, E>(a, ka, s); break;
    case 128: e = run_decode_gate<128, E>(a, ka, s); break;
  }
  if (e != hipSuccess) return e;
  if (a.conv_q) {  // after the step has read the state
    hipLaunchKernelGGL(conv_state_advance_kernel<E>, dim3((unsigned)((size_t)a.N * a.H)), dim3(256), 0, s,
                       reinterpret_cast<const E *>(a.q), reinterpret_cast<const E *>(a.k),
                       reinterpret_cast<const E *>(a.v), reinterpret_cast<E *>(a.conv_state), a.H, a.dk, a.dv, a.Tk,
                       (unsigned)((size_t)a.N * a.H));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_out_norm_gate(a.o, a.out_gate, a.norm_w, a.norm_eps, a.H, (long long)a.N * a.Tk, a.dv, a.bf16, s);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if ((size_t)a.N * a.H == 0) return hipSuccess;
  if (a.Tk == 0) {  // no token: the state passes through
    if (a.S == a.S_in) return hipSuccess;
    return hipMemcpyAsync(a.S, a.S_in, (size_t)a.N * a.H * a.dv * a.dk * sizeof(float), hipMemcpyDeviceToDevice,
                          stream);
  }
  return a.bf16 ? run_decode<bf16>(a, stream) : run_decode<float>(a, stream);
}

}  // namespace kda
