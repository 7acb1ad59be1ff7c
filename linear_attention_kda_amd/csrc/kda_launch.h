// kda_launch.h -- internal interface between the C ABI (kda_api.cpp) and the
// kernel launchers (kda_prefill.hip, kda_decode.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

constexpr int kChunkTokens = 64;

// One record per (chunk, head) of the prefill workspace, written by the
// chunk-prep kernel and read by the scan kernel.  Element type E is the dtype
// of q/k/v (2 or 4 bytes).  The five matrices are stored as A operands of the
// 16x16 matrix-core products, in fragment order (see frag_index in
// kda_prefill.hip): each lane's share of a 16-row x slab tile is 16 (or 8)
// contiguous bytes.  Offsets in bytes.
struct ChunkRecordLayout {
  size_t kh;    // k_i D_{0:i}          rows i (64),  K = d_k
  size_t qh;    // q_i D_{0:i}          rows i (64),  K = d_k
  size_t ktt;   // k_j D_{j+1:63}       rows c (d_k), K = 64 tokens (transposed)
  size_t tb;    // (I + R)^{-1} Diag(beta), rows i (64), K = 64, lower triangle (see tri_*)
  size_t aqk;   // scaled causal q-k scores incl. diagonal, rows i, K = 64, lower triangle
  size_t p63;   // [dk] fp32 whole-chunk decay D_{0:63}
  size_t bytes; // record size (multiple of 1024)
};

// The two lower-triangular 64 x 64 operands (Tb and A) keep, for each 16-row
// tile I, only the k-slabs that hold a column at or left of the diagonal:
// slabs of 32 columns for 2-byte elements, 16 for 4-byte ones, one 1 KiB
// fragment (64 lanes x 16 bytes) per (tile, slab).  The slabs of tile I start
// at fragment tri_slab0(I).
constexpr int tri_slab_width(int esize) { return esize == 2 ? 32 : 16; }
constexpr int tri_slabs(int I, int esize) { return (16 * (I + 1) + tri_slab_width(esize) - 1) / tri_slab_width(esize); }
constexpr int tri_slab0(int I, int esize) { return I == 0 ? 0 : tri_slab0(I - 1, esize) + tri_slabs(I - 1, esize); }
constexpr size_t tri_bytes(int esize) { return (size_t)tri_slab0(4, esize) * 1024; }

inline ChunkRecordLayout chunk_record_layout(int dk, int esize) {
  ChunkRecordLayout L;
  L.kh = 0;
  L.qh = L.kh + (size_t)64 * dk * esize;
  L.ktt = L.qh + (size_t)64 * dk * esize;
  L.tb = L.ktt + (size_t)64 * dk * esize;
  L.aqk = L.tb + tri_bytes(esize);
  L.p63 = L.aqk + tri_bytes(esize);
  size_t end = L.p63 + (size_t)dk * sizeof(float);
  L.bytes = (end + 1023) / 1024 * 1024;
  return L;
}

// Control words at the start of every prefill workspace (kCtlWords int32):
// the schedule the last call ran (a kSchedule* value other than auto) and
// the overlapped schedule's error bits, read back by kda_chunk_fwd_status,
// then that schedule's per-XCD task counters of the prep and of the scan.
constexpr int kCtlSchedule = 0, kCtlError = 1, kCtlPrepNext = 8, kCtlScanNext = 16, kCtlWords = 64;
constexpr size_t kCtlBytes = kCtlWords * sizeof(int32_t);
// error bits: a ready-flag wait timed out / a record came from another XCD
constexpr int kSchedErrTimeout = 1, kSchedErrXcd = 2;

// Split-sequence prefill (a dense batch of few units at d_k = d_v = 128,
// bf16): each sequence is cut into G segments of cps chunks (the last one
// shorter).  A first scan pass gives the affine map of the state over every
// segment but the last (S_end = S_start M + X), a small pass chains the maps
// into each segment's start state, and the ordinary scan then runs all
// segments at once.  The pass over the maps costs about as much per chunk as
// the scan, so the split pays only when the units leave most of the chip
// idle: G is chosen by a cost model in scan steps (the map pass at 0.8 of a
// scan step with two compute waves per workgroup, or half the workgroups at
// 1.3 times that with four; whole waves of 256 workgroups; a chained segment
// at about 1.2 scan steps), and taken automatically when it saves a quarter
// of the sequential chain.
struct SplitPlan {
  int G = 1;          // segments per sequence (1: no split)
  int cps = 0;        // chunks per segment (all but the last)
  bool worth = false; // the automatic schedule takes it
  int map_cw = 2;     // compute waves (16 columns each) per map-scan workgroup: 2 or 4
};
constexpr int kSplitMinChunks = 16;  // chunks per segment, at least
constexpr int kSplitMaxSegments = 16;
inline SplitPlan split_plan(int B, int T, int H, int dk, int dv, int esize) {
  SplitPlan sp;
  if (dk != 128 || dv != 128 || esize != 2 || B <= 0 || T <= 0) return sp;
  const long long units = (long long)B * H, nct = ((long long)T + kChunkTokens - 1) / kChunkTokens;
  const long long wg_scan = units * (dv / 32), wg_map = units * ((dv + dk) / 32);
  double best = (double)nct;  // the sequential chain, in scan steps
  for (int G = 2; G <= kSplitMaxSegments; ++G) {
    const long long cps = (nct + G - 1) / G;
    if (cps < kSplitMinChunks) break;
    if ((G - 1) * cps >= nct) continue;  // the last segment would be empty
    // maps: with two compute waves per workgroup a state-only step costs
    // about 0.8 of a scan step; with four (half the workgroups, twice the
    // columns each) about 1.3 times that, which pays only once the
    // two-wave maps need more than one round of 256 workgroups
    const long long wg2 = (G - 1) * wg_map, wg4 = wg2 / 2;
    const double map2 = (double)((wg2 + 255) / 256) * cps * 0.8;
    const double map4 = (double)((wg4 + 255) / 256) * cps * 0.8 * 1.3;
    const bool four = wg2 > 256 && map4 < map2;
    const double waves3 = (double)((G * wg_scan + 255) / 256);
    const double est = (four ? map4 : map2) + waves3 * cps + 1.2 * (G - 1);
    if (est < best) {
      best = est;
      sp.G = G;
      sp.cps = (int)cps;
      sp.map_cw = four ? 4 : 2;
    }
  }
  sp.worth = sp.G > 1 && best < 0.75 * (double)nct;
  return sp;
}

// Workspace = [control words] [index tables (packed batches only)]
//             [chunk records] [ready flags (dense batches only)]
//             [split-sequence buffers (dense batches a split can serve)].
struct WorkspacePlan {
  int n_seq;           // sequences
  long long max_chunks;// chunk slots (dense: exact count)
  size_t tables;       // byte offset of the index tables
  size_t tables_bytes; // 0 for dense batches
  size_t records;      // byte offset of the chunk records
  size_t record_bytes;
  size_t ready;        // byte offset of the ready flags (dense only)
  size_t ready_bytes;  // one int32 per record slot, 0 for packed batches
  size_t total;
  // int32 table offsets (in elements from `tables`), packed only
  size_t seq_tok0, seq_chunk0, chunk_t0, chunk_len, chunk_s0, seq_order;
  // split-sequence prefill (split.G > 1 only): byte offsets of the segment
  // tables (B G + 1 token offsets, then B G + 1 chunk offsets, int32), the
  // maps ([B (G-1) H] x (d_v + d_k) x d_k fp32: X rows, then M^T rows), the
  // segment start states and the segments' end states ([B G H] x d_v x d_k
  // fp32 each)
  SplitPlan split;
  size_t sp_tables, sp_maps, sp_start, sp_end;
};

// dv = 0: no split-sequence buffers (the no-allocation entry point).
inline WorkspacePlan plan_workspace(bool packed, int B, int T, int H, int dk,
                                    int N, int esize, int dv = 0) {
  WorkspacePlan P{};
  ChunkRecordLayout L = chunk_record_layout(dk, esize);
  P.record_bytes = L.bytes;
  P.tables = kCtlBytes;
  if (packed) {
    P.n_seq = N;
    P.max_chunks = ((long long)T + kChunkTokens - 1) / kChunkTokens + N;
    P.seq_tok0 = 0;
    P.seq_chunk0 = P.seq_tok0 + (size_t)N + 1;
    P.chunk_t0 = P.seq_chunk0 + (size_t)N + 1;
    P.chunk_len = P.chunk_t0 + (size_t)P.max_chunks;
    P.chunk_s0 = P.chunk_len + (size_t)P.max_chunks;
    P.seq_order = P.chunk_s0 + (size_t)P.max_chunks;
    size_t n_int = P.seq_order + (size_t)N;
    P.tables_bytes = (n_int * sizeof(int32_t) + 255) / 256 * 256;
  } else {
    P.n_seq = B;
    P.max_chunks = (long long)B * (((long long)T + kChunkTokens - 1) / kChunkTokens);
    P.tables_bytes = 0;
  }
  P.records = P.tables + P.tables_bytes;
  P.ready = P.records + (size_t)P.max_chunks * H * P.record_bytes;
  P.ready_bytes = packed ? 0 : ((size_t)P.max_chunks * H * sizeof(int32_t) + 255) / 256 * 256;
  P.total = P.ready + P.ready_bytes;
  if (!packed && dv > 0) P.split = split_plan(B, T, H, dk, dv, esize);
  if (P.split.G > 1) {
    const size_t G = (size_t)P.split.G, state = (size_t)dv * dk * sizeof(float);
    P.sp_tables = P.total;
    P.sp_maps = P.sp_tables + ((2 * ((size_t)B * G + 1) * sizeof(int32_t) + 255) / 256 * 256);
    P.sp_start = P.sp_maps + (size_t)B * (G - 1) * H * (size_t)(dv + dk) * dk * sizeof(float);
    P.sp_end = P.sp_start + (size_t)B * G * H * state;
    P.total = P.sp_end + (size_t)B * G * H * state;
  }
  return P;
}

// gate forms (kda_gate): gates, their logarithms or softplus logits, one per
// key channel or one per token and head, or none
constexpr int kGateChannel = 0, kGateScalar = 1, kGateNone = 2, kGateLogChannel = 3, kGateLogScalar = 4,
              kGateSoftplusChannel = 5, kGateSoftplusScalar = 6;
// gate forms that read one value per key channel / one per token and head
constexpr bool gate_per_channel(int g) {
  return g == kGateChannel || g == kGateLogChannel || g == kGateSoftplusChannel;
}
constexpr bool gate_per_token(int g) { return g == kGateScalar || g == kGateLogScalar || g == kGateSoftplusScalar; }
constexpr bool gate_is_log(int g) { return g == kGateLogChannel || g == kGateLogScalar; }
constexpr bool gate_is_softplus(int g) { return g == kGateSoftplusChannel || g == kGateSoftplusScalar; }

// input activations applied on load (kda_input_act bits)
constexpr unsigned kActQK = 1;    // q, k <- L2-normalised SiLU, per token and head
constexpr unsigned kActBeta = 2;  // beta <- sigmoid(beta)

// Short causal convolution of q, k and v (kda_module_ops): this many taps
// per channel, the last one on the current token.
constexpr int kConvTaps = 4;

// Prefill schedules (kda_set_schedule): automatic, always prep then scan,
// prep and scan overlapped whenever the shapes allow it, or split-sequence
// whenever the shapes allow it.
constexpr int kScheduleAuto = 0, kScheduleTwoPhase = 1, kScheduleOverlap = 2, kScheduleSplit = 3;

// Default bound on one ready-flag wait of the overlapped scan: 2^27 ticks of
// the 100 MHz real-time counter, about 1.3 s.
constexpr long long kDefaultWaitTicks = 1ll << 27;

struct PrefillArgs {
  int schedule;               // kSchedule*
  long long wait_ticks;       // bound on one ready-flag wait (overlapped schedule)
  const void *q, *k, *v;
  const float *alpha, *beta, *S0;
  int gate;
  unsigned act;               // kAct* bits
  const int32_t *cu_seqlens;  // device, or null for a dense batch
  void *o;
  float *S_final;
  char *ws;                   // workspace base
  WorkspacePlan plan;
  int B, T, H, dk, dv;
  float scale;
  bool bf16;
  // module operations around the method (kda_module_ops), all optional:
  // depthwise causal convolution taps [H, d, kConvTaps] of q, k and v (all
  // three or none), and the output's RMS norm gains [d_v] and gate logits
  // (same layout and type as o)
  const float *conv_q, *conv_k, *conv_v;
  const float *norm_w;
  const void *out_gate;
  float norm_eps;
  void *conv_state;  // with the convolution: the last three raw tokens per (sequence, head), written (optional)
};

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

// Destroys the internal streams and events of the overlapped schedule on
// every device (kda_release); idempotent.
void release_overlap();

// The no-allocation prefill's device scratch: a static array of this many
// bytes per device, whose address on the current device (looked up once per
// device with hipGetSymbolAddress) goes to *ptr.
constexpr size_t kScratchBytes = (size_t)64 << 20;
hipError_t scratch_address(void **ptr);

// Optional value checks (see kda_set_validation).  Bits of the result:
constexpr unsigned kValidateAlpha = 1, kValidateBeta = 2, kValidateKey = 4, kValidateOffsets = 8;
constexpr float kValidateKeyTol = 1.0f / 64;  // | |k|^2 - 1 | allowed
struct ValidateArgs {
  const float *alpha;   // null when the gate form reads none
  size_t n_alpha;
  int gate_range;       // 0: gates in [0, 1]; 1: log gates <= 0; 2: any number (logits)
  const float *beta;
  size_t n_beta;
  bool beta_logits;     // beta is a logit (sigmoid on load): any number
  const void *k;
  size_t n_krows;       // 0 when k is normalised on load
  int dk;
  bool k_bf16;
  const int32_t *cu;    // null for a dense batch
  int n_seq, total;
};
// Runs the checks on `stream`, waits for them and returns the violated
// conditions in *bits (0: none).  Synchronises the stream.
hipError_t run_validation(const ValidateArgs &v, hipStream_t stream, unsigned *bits);

struct DecodeArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  int gate;
  unsigned act;       // kAct* bits
  const float *S_in;  // state read
  float *S;           // state written (may be S_in)
  void *o;
  int N, H, dk, dv;
  int Tk;             // tokens per sequence (1 for a single step)
  float scale;
  bool bf16;
  // module operations (kda_module_ops), optional: convolution taps of q, k
  // and v with the convolution state [N, H, 3, 2 d_k + d_v] (read, then
  // replaced), output norm gains and gate logits
  const float *conv_q, *conv_k, *conv_v;
  void *conv_state;
  const float *norm_w;
  const void *out_gate;
  float norm_eps;
};

// The output norm and gate pass of the module operations over n_tok x H rows
// of d_v values of o (gate logits of the same layout), on `stream`.
hipError_t launch_out_norm_gate(void *o, const void *gate, const float *w, float eps, int H, long long n_tok, int dv,
                                bool is_bf16, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);

}  // namespace kda
