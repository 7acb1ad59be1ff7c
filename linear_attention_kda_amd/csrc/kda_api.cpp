// kda_api.cpp -- the exported C ABI (include/kda.h): argument validation,
// workspace sizing and dispatch to the HIP launchers.  Host code only; every
// step of the computation runs in the kernels of kda_prefill.hip and
// kda_decode.hip.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstdint>
#include <cstdlib>
#include <mutex>

#include "kda_launch.h"

namespace {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
// The scan stores a chunk's outputs through one buffer range of 32-bit size:
// 64 token rows of all heads' values, at most 4 bytes each.
bool width_ok(int H, int d_v) { return (size_t)H * d_v * 64 * 4 <= (size_t)INT32_MAX; }
constexpr unsigned kActAll = KDA_ACT_QK_SILU_L2NORM | KDA_ACT_BETA_SIGMOID;
bool valid_gate(kda_gate g) {
  return g == KDA_GATE_CHANNEL || g == KDA_GATE_SCALAR || g == KDA_GATE_NONE || g == KDA_GATE_LOG_CHANNEL ||
         g == KDA_GATE_LOG_SCALAR || g == KDA_GATE_SOFTPLUS_CHANNEL || g == KDA_GATE_SOFTPLUS_SCALAR;
}
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void *p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

float default_scale(float scale, int dk) {
  return scale > 0.f ? scale : 1.0f / std::sqrt((float)dk);
}

// Value checks: off unless KDA_VALIDATE is set to a nonzero integer in the
// environment when the library is loaded, or kda_set_validation(1) is called.
std::atomic<int> g_validate{[] {
  const char *e = std::getenv("KDA_VALIDATE");
  return e && std::atoi(e) != 0 ? 1 : 0;
}()};

// Prefill schedule (kda_set_schedule): KDA_SCHEDULE in the environment at
// load time, else automatic.
std::atomic<int> g_schedule{[] {
  const char *e = std::getenv("KDA_SCHEDULE");
  const int v = e ? std::atoi(e) : 0;
  return v == kda::kScheduleTwoPhase || v == kda::kScheduleOverlap || v == kda::kScheduleSplit ? v
                                                                                               : kda::kScheduleAuto;
}()};

// Bound on the overlapped scan's ready-flag waits (kda_set_sched_wait_limit).
std::atomic<long long> g_wait_ticks{kda::kDefaultWaitTicks};

// One value check at a time in the process: the kernel reports through one
// device word per device, cleared before and read back after the check.
std::mutex g_validate_mu;

bool capturing(hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone;
}

// Runs the device checks when they are on.  KDA_OK when off or clean.
kda_status check_values(const float *alpha, size_t n_alpha, kda_gate gate, const float *beta, size_t n_beta,
                        unsigned act, const void *k, size_t n_krows, int d_k, kda_dtype dtype, const int32_t *cu,
                        int n_seq, int total, hipStream_t stream) {
  if (!g_validate.load(std::memory_order_relaxed)) return KDA_OK;
  // the check waits for the stream, which a stream being captured cannot do
  if (capturing(stream)) return KDA_ERR_STREAM_CAPTURE;
  const int range = kda::gate_is_log(gate) ? 1 : kda::gate_is_softplus(gate) ? 2 : 0;
  // keys normalised on load need no unit norm
  kda::ValidateArgs v{alpha, alpha ? n_alpha : 0, range, beta, n_beta, (act & kda::kActBeta) != 0, k,
                      (act & kda::kActQK) ? 0 : n_krows, d_k, dtype == KDA_BF16, cu, n_seq, total};
  unsigned bits = 0;
  std::lock_guard<std::mutex> lock(g_validate_mu);
  if (kda::run_validation(v, stream, &bits) != hipSuccess) return KDA_ERR_HIP;
  return bits ? KDA_ERR_INVALID_VALUE : KDA_OK;
}

// The no-allocation prefill (kda_chunk_fwd_noalloc): the same kernels, two-
// phase, on the library's static device scratch instead of a caller's
// workspace.  A packed batch, or a dense batch whose whole plan fits, runs as
// one call; a larger dense batch runs one sequence at a time in segments of
// whole chunks, each segment starting from the state the previous one left
// in S_final (identical arithmetic: a chunk boundary is a chunk boundary).
// No value checks (they would copy to the host and wait).
kda_status chunk_fwd_scratch(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                             const float *beta, unsigned input_act, const float *S0, const int32_t *cu_seqlens, int N,
                             int B, int T, int H, int d_k, int d_v, float scale, kda_dtype dtype, void *o,
                             float *S_final, hipStream_t stream) {
  const int es = dtype == KDA_BF16 ? 2 : 4;
  const bool packed = cu_seqlens != nullptr;
  const kda::WorkspacePlan whole = kda::plan_workspace(packed, B, T, H, d_k, N, es);
  char *scratch = nullptr;
  if (kda::scratch_address(reinterpret_cast<void **>(&scratch)) != hipSuccess || !scratch) return KDA_ERR_HIP;
  kda::PrefillArgs a{};
  a.schedule = kda::kScheduleTwoPhase;
  a.wait_ticks = kda::kDefaultWaitTicks;
  a.gate = (int)gate;
  a.act = input_act;
  a.H = H;
  a.dk = d_k;
  a.dv = d_v;
  a.scale = default_scale(scale, d_k);
  a.bf16 = dtype == KDA_BF16;
  a.ws = scratch;
  if (packed || T == 0 || whole.total <= kda::kScratchBytes) {
    if (whole.total > kda::kScratchBytes) return KDA_ERR_TOO_LARGE;
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.beta = beta; a.S0 = S0; a.cu_seqlens = cu_seqlens;
    a.o = o; a.S_final = S_final; a.plan = whole; a.B = B; a.T = T;
    return kda::launch_prefill(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
  }
  // chunks per segment: the most that fit, for one sequence
  const int nct = (T + kda::kChunkTokens - 1) / kda::kChunkTokens;
  int seg = nct;
  while (seg > 0 && kda::plan_workspace(false, 1, seg * kda::kChunkTokens, H, d_k, 1, es).total > kda::kScratchBytes)
    seg = seg > 64 ? seg / 2 : seg - 1;
  if (seg == 0) return KDA_ERR_TOO_LARGE;
  const size_t tok_q = (size_t)H * d_k, tok_v = (size_t)H * d_v;
  const size_t tok_a = kda::gate_per_channel(gate) ? tok_q : kda::gate_per_token(gate) ? (size_t)H : 0;
  const size_t state = (size_t)H * d_v * d_k;
  for (int b = 0; b < B; ++b) {
    for (int c0 = 0; c0 < nct; c0 += seg) {
      const size_t t0 = (size_t)b * T + (size_t)c0 * kda::kChunkTokens;
      const int Ts = (int)std::min<long long>((long long)seg * kda::kChunkTokens, (long long)T - (long long)c0 * kda::kChunkTokens);
      a.q = static_cast<const char *>(q) + t0 * tok_q * es;
      a.k = static_cast<const char *>(k) + t0 * tok_q * es;
      a.v = static_cast<const char *>(v) + t0 * tok_v * es;
      a.alpha = alpha ? alpha + t0 * tok_a : nullptr;
      a.beta = beta + t0 * H;
      a.o = static_cast<char *>(o) + t0 * tok_v * es;
      a.S_final = S_final + (size_t)b * state;
      // the first segment starts from S0 (or zeros), every later one from the
      // state the previous segment wrote (S_final in place)
      a.S0 = c0 == 0 ? (S0 ? S0 + (size_t)b * state : nullptr) : a.S_final;
      a.cu_seqlens = nullptr;
      a.B = 1;
      a.T = Ts;
      a.plan = kda::plan_workspace(false, 1, Ts, H, d_k, 1, es);
      if (kda::launch_prefill(a, stream) != hipSuccess) return KDA_ERR_HIP;
    }
  }
  return KDA_OK;
}

// kda_chunk_fwd_module (ops may be null), and with noalloc the variant of
// kda_chunk_fwd_ex on the library's static scratch (kda_chunk_fwd_noalloc;
// workspace and ops are then ignored).
kda_status chunk_fwd_impl(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                          const float *beta, unsigned input_act, const kda_module_ops *ops, const float *S0,
                          const int32_t *cu_seqlens, int N, int B, int T, int H, int d_k, int d_v, float scale,
                          kda_dtype dtype, void *o, float *S_final, void *workspace, size_t workspace_bytes,
                          hipStream_t stream, bool noalloc) {
  if (noalloc) {
    workspace = nullptr;
    workspace_bytes = 0;
    ops = nullptr;
  }
  const kda_module_ops mo = ops ? *ops : kda_module_ops{nullptr, nullptr, nullptr, nullptr, 0.f, nullptr, nullptr};
  const bool conv = mo.conv_q || mo.conv_k || mo.conv_v;
  if (!valid_gate(gate)) return KDA_ERR_UNSUPPORTED_GATE;
  if (input_act & ~kActAll) return KDA_ERR_UNSUPPORTED_ACT;
  if (conv && !(mo.conv_q && mo.conv_k && mo.conv_v)) return KDA_ERR_NULL_ARG;
  if (conv && !(input_act & KDA_ACT_QK_SILU_L2NORM)) return KDA_ERR_UNSUPPORTED_ACT;
  if (mo.norm_weight && !(mo.norm_eps >= 0.f)) return KDA_ERR_BAD_SHAPE;
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED_DTYPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED_DIM;
  if (B < 0 || T < 0 || H <= 0 || !width_ok(H, d_v)) return KDA_ERR_BAD_SHAPE;
  const bool packed = cu_seqlens != nullptr;
  if (packed) {
    if (B != 1) return KDA_ERR_VARLEN_REQUIRES_B1;
    if (N < 0) return KDA_ERR_BAD_SHAPE;
  } else {
    N = B;
  }
  const size_t es = dtype == KDA_BF16 ? 2 : 4;
  const size_t ntok = (size_t)B * T;
  const size_t qk_bytes = ntok * H * d_k * es, v_bytes = ntok * H * d_v * es;
  const size_t a_bytes = kda::gate_per_channel(gate) ? ntok * H * d_k * sizeof(float)
                         : kda::gate_per_token(gate) ? ntok * H * sizeof(float) : 0;
  const size_t b_bytes = ntok * H * sizeof(float);
  const size_t s_bytes = (size_t)N * H * d_v * d_k * sizeof(float);
  if (gate == KDA_GATE_NONE) alpha = nullptr;
  if (ntok > 0 && (!q || !k || !v || (a_bytes && !alpha) || !beta || !o)) return KDA_ERR_NULL_ARG;
  if (s_bytes > 0 && !S_final) return KDA_ERR_NULL_ARG;
  if (ntok > (size_t)INT32_MAX) return KDA_ERR_BAD_SHAPE;
  const void *ptrs[] = {q,         k,         v,         alpha,          beta,        S0,           cu_seqlens,
                        o,         S_final,   workspace, mo.conv_q,      mo.conv_k,   mo.conv_v,    mo.norm_weight,
                        mo.out_gate, mo.conv_state};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;

  const kda::WorkspacePlan plan = kda::plan_workspace(packed, B, T, H, d_k, N, (int)es, noalloc ? 0 : d_v);
  if (!noalloc && plan.total > 0 && (!workspace || workspace_bytes < plan.total)) return KDA_ERR_WORKSPACE_TOO_SMALL;

  {
    // Every output (o, S_final) and the workspace must be disjoint from each
    // other and from every input; S_final may only be S0 itself (in place).
    const Range ro = range_of(o, ntok > 0 ? ntok * H * d_v * es : 0);
    const Range rs = range_of(S_final, s_bytes), rw = range_of(workspace, noalloc ? 0 : plan.total);
    const size_t wq_bytes = (size_t)H * d_k * kda::kConvTaps * sizeof(float);
    const size_t wv_bytes = (size_t)H * d_v * kda::kConvTaps * sizeof(float);
    const Range ins[] = {range_of(q, ntok > 0 ? qk_bytes : 0), range_of(k, ntok > 0 ? qk_bytes : 0),
                         range_of(v, ntok > 0 ? v_bytes : 0), range_of(alpha, alpha && ntok > 0 ? a_bytes : 0),
                         range_of(beta, ntok > 0 ? b_bytes : 0),
                         range_of(cu_seqlens, packed ? ((size_t)N + 1) * sizeof(int32_t) : 0),
                         range_of(mo.conv_q, mo.conv_q ? wq_bytes : 0), range_of(mo.conv_k, mo.conv_k ? wq_bytes : 0),
                         range_of(mo.conv_v, mo.conv_v ? wv_bytes : 0),
                         range_of(mo.norm_weight, mo.norm_weight ? (size_t)d_v * sizeof(float) : 0),
                         range_of(mo.out_gate, mo.out_gate && ntok > 0 ? v_bytes : 0)};
    for (const Range &r : ins)
      if (overlaps(ro, r) || overlaps(rs, r) || overlaps(rw, r)) return KDA_ERR_ALIAS;
    const Range rs0 = range_of(S0, S0 ? s_bytes : 0);
    if (overlaps(ro, rs) || overlaps(ro, rw) || overlaps(rs, rw) || overlaps(ro, rs0) || overlaps(rw, rs0))
      return KDA_ERR_ALIAS;
    if (S0 && S0 != S_final && overlaps(rs, rs0)) return KDA_ERR_ALIAS;
    // the final convolution state (an output, with the convolution) overlaps nothing
    if (conv && mo.conv_state) {
      const Range rcs = range_of(mo.conv_state, (size_t)N * H * 3 * (2 * (size_t)d_k + d_v) * es);
      for (const Range &r : ins)
        if (overlaps(rcs, r)) return KDA_ERR_ALIAS;
      if (overlaps(rcs, ro) || overlaps(rcs, rs) || overlaps(rcs, rw) || overlaps(rcs, rs0)) return KDA_ERR_ALIAS;
    }
  }
  if (N == 0) return KDA_OK;
  if (noalloc)
    return chunk_fwd_scratch(q, k, v, alpha, gate, beta, input_act, S0, cu_seqlens, N, B, T, H, d_k, d_v, scale, dtype,
                             o, S_final, stream);
  if (const kda_status st = check_values(alpha, a_bytes / sizeof(float), gate, beta, ntok * H, input_act, k,
                                         ntok * H, d_k, dtype, cu_seqlens, N, T, stream))
    return st;

  kda::PrefillArgs a{};
  a.schedule = g_schedule.load(std::memory_order_relaxed);
  a.wait_ticks = g_wait_ticks.load(std::memory_order_relaxed);
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.gate = (int)gate;
  a.act = input_act;
  a.beta = beta;
  a.S0 = S0;
  a.cu_seqlens = cu_seqlens;
  a.o = o;
  a.S_final = S_final;
  a.ws = static_cast<char *>(workspace);
  a.plan = plan;
  a.B = B;
  a.T = T;
  a.H = H;
  a.dk = d_k;
  a.dv = d_v;
  a.scale = default_scale(scale, d_k);
  a.bf16 = dtype == KDA_BF16;
  if (conv) {
    a.conv_q = mo.conv_q;
    a.conv_k = mo.conv_k;
    a.conv_v = mo.conv_v;
    a.conv_state = mo.conv_state;
  }
  a.norm_w = mo.norm_weight;
  a.norm_eps = mo.norm_eps;
  a.out_gate = mo.out_gate;
  return kda::launch_prefill(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL_ARG: return "a required pointer is NULL";
    case KDA_ERR_BAD_SHAPE: return "a size is negative or the sizes are inconsistent";
    case KDA_ERR_UNSUPPORTED_DIM: return "d_k and d_v must each be 16, 32, 64 or 128";
    case KDA_ERR_UNSUPPORTED_DTYPE: return "dtype must be KDA_F32 or KDA_BF16";
    case KDA_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "workspace is smaller than kda_chunk_fwd_workspace_size()";
    case KDA_ERR_VARLEN_REQUIRES_B1: return "cu_seqlens requires B == 1";
    case KDA_ERR_ALIAS: return "an output overlaps an input, another output or the workspace";
    case KDA_ERR_HIP: return "the HIP runtime reported an error";
    case KDA_ERR_UNSUPPORTED_GATE: return "gate must be a kda_gate value (channel, scalar, none, log channel, log scalar)";
    case KDA_ERR_INVALID_VALUE:
      return "an input value is out of range (gate or beta outside [0, 1], a key of norm not 1, or bad cu_seqlens)";
    case KDA_ERR_UNSUPPORTED_ACT: return "input_act has bits that are not kda_input_act flags";
    case KDA_ERR_STREAM_CAPTURE:
      return "the stream is being captured into a graph, and this call has to wait for the device";
    case KDA_ERR_TOO_LARGE:
      return "the sizes need more device scratch than the no-allocation entry point holds";
  }
  return "unknown status";
}

int kda_set_validation(int enable) {
  if (enable < 0) return g_validate.load();
  return g_validate.exchange(enable ? 1 : 0);
}

kda_status kda_chunk_fwd_status(const void *workspace, hipStream_t stream, int *schedule, unsigned *errors) {
  if (!workspace) return KDA_ERR_NULL_ARG;
  if (!aligned16(workspace)) return KDA_ERR_MISALIGNED;
  if (capturing(stream)) return KDA_ERR_STREAM_CAPTURE;
  int32_t words[2] = {0, 0};
  static_assert(kda::kCtlSchedule == 0 && kda::kCtlError == 1, "status words first");
  if (hipMemcpyAsync(words, workspace, sizeof(words), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return KDA_ERR_HIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return KDA_ERR_HIP;
  if (schedule) *schedule = words[0];
  if (errors) *errors = (unsigned)words[1];
  return KDA_OK;
}

void kda_release(void) { kda::release_overlap(); }

long long kda_set_sched_wait_limit(long long ticks) {
  if (ticks < 0) return g_wait_ticks.load();
  return g_wait_ticks.exchange(ticks);
}

int kda_set_schedule(int schedule) {
  if (schedule != KDA_SCHEDULE_AUTO && schedule != KDA_SCHEDULE_TWO_PHASE && schedule != KDA_SCHEDULE_OVERLAP &&
      schedule != KDA_SCHEDULE_SPLIT)
    return -1;
  return g_schedule.exchange(schedule);
}

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int d_k, int d_v, int N, kda_dtype dtype) {
  if (B < 0 || T < 0 || H <= 0 || !dim_ok(d_k) || !dim_ok(d_v) || !width_ok(H, d_v)) return 0;
  if (dtype != KDA_F32 && dtype != KDA_BF16) return 0;
  const int esize = dtype == KDA_BF16 ? 2 : 4;
  size_t need = kda::plan_workspace(false, B, T, H, d_k, B, esize, d_v).total;
  if (B == 1 && N >= 0) {  // may be a packed batch of N sequences
    const size_t pk = kda::plan_workspace(true, 1, T, H, d_k, N, esize).total;
    if (pk > need) need = pk;
  }
  return need;
}

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                         const float *S0, const int32_t *cu_seqlens, int N, int B, int T, int H, int d_k,
                         int d_v, float scale, kda_dtype dtype, void *o, float *S_final, void *workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return kda_chunk_fwd_gated(q, k, v, alpha, KDA_GATE_CHANNEL, beta, S0, cu_seqlens, N, B, T, H, d_k, d_v, scale,
                             dtype, o, S_final, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_gated(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                               const float *beta, const float *S0, const int32_t *cu_seqlens, int N, int B, int T,
                               int H, int d_k, int d_v, float scale, kda_dtype dtype, void *o, float *S_final,
                               void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return kda_chunk_fwd_ex(q, k, v, alpha, gate, beta, KDA_ACT_NONE, S0, cu_seqlens, N, B, T, H, d_k, d_v, scale,
                          dtype, o, S_final, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                            const float *beta, unsigned input_act, const float *S0, const int32_t *cu_seqlens, int N,
                            int B, int T, int H, int d_k, int d_v, float scale, kda_dtype dtype, void *o,
                            float *S_final, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, alpha, gate, beta, input_act, nullptr, S0, cu_seqlens, N, B, T, H, d_k, d_v, scale,
                        dtype, o, S_final, workspace, workspace_bytes, stream, false);
}

kda_status kda_chunk_fwd_module(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                                const float *beta, unsigned input_act, const kda_module_ops *ops, const float *S0,
                                const int32_t *cu_seqlens, int N, int B, int T, int H, int d_k, int d_v, float scale,
                                kda_dtype dtype, void *o, float *S_final, void *workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, alpha, gate, beta, input_act, ops, S0, cu_seqlens, N, B, T, H, d_k, d_v, scale,
                        dtype, o, S_final, workspace, workspace_bytes, stream, false);
}

kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                                 const float *beta, unsigned input_act, const float *S0, const int32_t *cu_seqlens,
                                 int N, int B, int T, int H, int d_k, int d_v, float scale, kda_dtype dtype, void *o,
                                 float *S_final, hipStream_t stream) {
  return chunk_fwd_impl(q, k, v, alpha, gate, beta, input_act, nullptr, S0, cu_seqlens, N, B, T, H, d_k, d_v, scale,
                        dtype, o, S_final, nullptr, 0, stream, true);
}

kda_status kda_decode_step(const void *q, const void *k, const void *v, const float *alpha, const float *beta,
                           float *S, int N, int H, int d_k, int d_v, float scale, kda_dtype dtype, void *o,
                           hipStream_t stream) {
  return kda_decode_step_gated(q, k, v, alpha, KDA_GATE_CHANNEL, beta, S, N, H, d_k, d_v, scale, dtype, o, stream);
}

kda_status kda_decode_step_gated(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                                 const float *beta, float *S, int N, int H, int d_k, int d_v, float scale,
                                 kda_dtype dtype, void *o, hipStream_t stream) {
  if (!valid_gate(gate)) return KDA_ERR_UNSUPPORTED_GATE;
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED_DTYPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED_DIM;
  if (N < 0 || H <= 0) return KDA_ERR_BAD_SHAPE;
  const size_t units = (size_t)N * H;
  if (units == 0) return KDA_OK;
  if (gate == KDA_GATE_NONE) alpha = nullptr;
  if (!q || !k || !v || (gate != KDA_GATE_NONE && !alpha) || !beta || !S || !o) return KDA_ERR_NULL_ARG;
  const void *ptrs[] = {q, k, v, alpha, beta, S, o};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
  const size_t a_bytes = kda::gate_per_channel(gate) ? units * d_k * sizeof(float)
                         : kda::gate_per_token(gate) ? units * sizeof(float) : 0;
  if (units > (size_t)INT32_MAX) return KDA_ERR_BAD_SHAPE;
  const size_t es = dtype == KDA_BF16 ? 2 : 4;
  // o and the state S (read and written) must not overlap each other or an input
  const Range ro = range_of(o, units * d_v * es), rs = range_of(S, units * d_v * d_k * sizeof(float));
  const Range ins[] = {range_of(q, units * d_k * es), range_of(k, units * d_k * es),
                       range_of(v, units * d_v * es), range_of(alpha, alpha ? a_bytes : 0),
                       range_of(beta, units * sizeof(float))};
  for (const Range &r : ins)
    if (overlaps(ro, r) || overlaps(rs, r)) return KDA_ERR_ALIAS;
  if (overlaps(ro, rs)) return KDA_ERR_ALIAS;
  if (const kda_status st = check_values(alpha, a_bytes / sizeof(float), gate, beta, units, 0, k, units, d_k,
                                         dtype, nullptr, 0, 0, stream))
    return st;

  kda::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.gate = (int)gate;
  a.act = 0;
  a.beta = beta;
  a.S_in = S;
  a.S = S;
  a.Tk = 1;
  a.o = o;
  a.N = N;
  a.H = H;
  a.dk = d_k;
  a.dv = d_v;
  a.scale = default_scale(scale, d_k);
  a.bf16 = dtype == KDA_BF16;
  return kda::launch_decode(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_tokens(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                             const float *beta, const float *S_in, float *S_out, int N, int Tk, int H, int d_k,
                             int d_v, float scale, kda_dtype dtype, void *o, hipStream_t stream) {
  return kda_decode_tokens_ex(q, k, v, alpha, gate, beta, KDA_ACT_NONE, S_in, S_out, N, Tk, H, d_k, d_v, scale,
                              dtype, o, stream);
}

kda_status kda_decode_tokens_module(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                                    const float *beta, unsigned input_act, const kda_module_ops *ops,
                                    const float *S_in, float *S_out, int N, int Tk, int H, int d_k, int d_v,
                                    float scale, kda_dtype dtype, void *o, hipStream_t stream) {
  const kda_module_ops mo = ops ? *ops : kda_module_ops{nullptr, nullptr, nullptr, nullptr, 0.f, nullptr, nullptr};
  const bool conv = mo.conv_q || mo.conv_k || mo.conv_v;
  if (!valid_gate(gate)) return KDA_ERR_UNSUPPORTED_GATE;
  if (input_act & ~kActAll) return KDA_ERR_UNSUPPORTED_ACT;
  if (conv && !(mo.conv_q && mo.conv_k && mo.conv_v && mo.conv_state)) return KDA_ERR_NULL_ARG;
  if (conv && !(input_act & KDA_ACT_QK_SILU_L2NORM)) return KDA_ERR_UNSUPPORTED_ACT;
  if (mo.norm_weight && !(mo.norm_eps >= 0.f)) return KDA_ERR_BAD_SHAPE;
  if (dtype != KDA_F32 && dtype != KDA_BF16) return KDA_ERR_UNSUPPORTED_DTYPE;
  if (!dim_ok(d_k) || !dim_ok(d_v)) return KDA_ERR_UNSUPPORTED_DIM;
  if (N < 0 || H <= 0 || Tk < 0) return KDA_ERR_BAD_SHAPE;
  const size_t units = (size_t)N * H;
  if (units == 0) return KDA_OK;
  if (units > (size_t)INT32_MAX || (size_t)Tk * units > (size_t)INT32_MAX) return KDA_ERR_BAD_SHAPE;
  const size_t toks = (size_t)Tk * units;
  if (gate == KDA_GATE_NONE) alpha = nullptr;
  if (!S_in || !S_out) return KDA_ERR_NULL_ARG;
  if (toks > 0 && (!q || !k || !v || (gate != KDA_GATE_NONE && !alpha) || !beta || !o)) return KDA_ERR_NULL_ARG;
  const void *ptrs[] = {q,         k,         v,         alpha,          beta,        S_in,         S_out, o,
                        mo.conv_q, mo.conv_k, mo.conv_v, mo.norm_weight, mo.out_gate, mo.conv_state};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_MISALIGNED;
  const size_t es = dtype == KDA_BF16 ? 2 : 4;
  const size_t a_bytes = kda::gate_per_channel(gate) ? toks * d_k * sizeof(float)
                         : kda::gate_per_token(gate) ? toks * sizeof(float) : 0;
  const size_t s_bytes = units * d_v * d_k * sizeof(float);
  // the state is updated in place or written to a disjoint buffer
  if (S_in != S_out && overlaps(range_of(S_in, s_bytes), range_of(S_out, s_bytes))) return KDA_ERR_ALIAS;
  // the convolution state (read and rewritten) must not overlap any other
  // argument; the module weights and gate logits (inputs) must not overlap
  // an output
  {
    // (a range of size 0 overlaps nothing)
    const Range rcs = range_of(mo.conv_state, conv ? units * 3 * (2 * (size_t)d_k + d_v) * es : 0);
    const Range ro = range_of(o, toks * d_v * es), rso = range_of(S_out, s_bytes);
    const Range rw[] = {range_of(mo.conv_q, conv ? (size_t)H * d_k * 4 * sizeof(float) : 0),
                        range_of(mo.conv_k, conv ? (size_t)H * d_k * 4 * sizeof(float) : 0),
                        range_of(mo.conv_v, conv ? (size_t)H * d_v * 4 * sizeof(float) : 0),
                        range_of(mo.norm_weight, mo.norm_weight ? (size_t)d_v * sizeof(float) : 0),
                        range_of(mo.out_gate, mo.out_gate ? toks * d_v * es : 0)};
    const Range args[] = {range_of(q, toks * d_k * es), range_of(k, toks * d_k * es),
                          range_of(v, toks * d_v * es), range_of(alpha, alpha ? a_bytes : 0),
                          range_of(beta, toks * sizeof(float)), range_of(S_in, s_bytes), rso, ro};
    for (const Range &r : args)
      if (overlaps(rcs, r)) return KDA_ERR_ALIAS;
    for (const Range &x : rw)
      if (overlaps(x, rcs) || overlaps(x, ro) || overlaps(x, rso)) return KDA_ERR_ALIAS;
  }
  if (toks > 0) {
    // o and S_out must not overlap each other or an input (S_out == S_in is
    // the in-place update, checked above)
    const Range ro = range_of(o, toks * d_v * es), rso = range_of(S_out, s_bytes);
    const Range ins[] = {range_of(q, toks * d_k * es), range_of(k, toks * d_k * es),
                         range_of(v, toks * d_v * es), range_of(alpha, alpha ? a_bytes : 0),
                         range_of(beta, toks * sizeof(float))};
    for (const Range &r : ins)
      if (overlaps(ro, r) || overlaps(rso, r)) return KDA_ERR_ALIAS;
    if (overlaps(ro, range_of(S_in, s_bytes)) || overlaps(ro, rso)) return KDA_ERR_ALIAS;
    if (const kda_status st = check_values(alpha, a_bytes / sizeof(float), gate, beta, toks, input_act, k, toks,
                                           d_k, dtype, nullptr, 0, 0, stream))
      return st;
  }

  kda::DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.gate = (int)gate;
  a.act = input_act;
  a.beta = beta;
  a.S_in = S_in;
  a.S = S_out;
  a.o = o;
  a.N = N;
  a.H = H;
  a.dk = d_k;
  a.dv = d_v;
  a.Tk = Tk;
  a.scale = default_scale(scale, d_k);
  a.bf16 = dtype == KDA_BF16;
  if (conv) {
    a.conv_q = mo.conv_q;
    a.conv_k = mo.conv_k;
    a.conv_v = mo.conv_v;
    a.conv_state = mo.conv_state;
  }
  a.norm_w = mo.norm_weight;
  a.norm_eps = mo.norm_eps;
  a.out_gate = mo.out_gate;
  return kda::launch_decode(a, stream) == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status kda_decode_tokens_ex(const void *q, const void *k, const void *v, const float *alpha, kda_gate gate,
                                const float *beta, unsigned input_act, const float *S_in, float *S_out, int N,
                                int Tk, int H, int d_k, int d_v, float scale, kda_dtype dtype, void *o,
                                hipStream_t stream) {
  return kda_decode_tokens_module(q, k, v, alpha, gate, beta, input_act, nullptr, S_in, S_out, N, Tk, H, d_k, d_v,
                                  scale, dtype, o, stream);
}

}  // extern "C"
