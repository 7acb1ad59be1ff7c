/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention (KDA) library.
 *
 * The operation.  Page "Kimi Delta Attention (KDA)" (brain.bigb.es), opening
 * update equation and section "KDA: a separate gate per key channel", defines
 * one head of KDA on a state S of shape d_v x d_k (keys to values; key
 * channels are the columns of S):
 *
 *     S~_t   = S_{t-1} Diag(alpha_t)          forget, alpha_t in [0,1]^{d_k}
 *     e_t    = beta_t (v_t - S~_t k_t)        predict and correct, beta_t in [0,1]
 *     S_t    = S~_t + e_t k_t^T               write
 *     o_t    = scale * S_t q_t                read, after the write
 *
 * with scale = d_k^{-1/2} by default and k_t of unit norm (a caller
 * precondition; the library does not normalise).  The same page, section
 * "Two schedules for one recurrence", states that a token-by-token schedule
 * and a chunkwise schedule reach identical states and outputs; kda_chunk_fwd
 * runs the chunkwise one (chunks of 64 tokens) and kda_decode_step the
 * token-by-token one.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers, owned by the caller.  The
 *    library allocates no device memory and keeps no pointer to caller
 *    memory after a call returns.  The one thing it keeps is per device:
 *    the first call that takes the overlapped prefill schedule (see
 *    kda_set_schedule) creates two internal streams and three events there,
 *    which stay until kda_release() (registered to run at process exit).
 *  - Layouts are dense row-major with the last dimension contiguous; every
 *    tensor pointer must be 16-byte aligned.
 *  - Calls are asynchronous on `stream` (0 = the null stream); results are
 *    valid once the stream reaches them.  No call synchronises the host.
 *  - dtype selects the element type of q, k, v and o (KDA_F32 or KDA_BF16).
 *    alpha, beta and every state tensor are always fp32.
 *  - d_k and d_v must each be one of 16, 32, 64, 128.
 *  - Errors are returned, never printed; nothing aborts.  By default only
 *    conditions the host can check are validated.  Values outside alpha,
 *    beta in [0,1], non-monotone cu_seqlens or a non-unit k are then not
 *    detected: the result is unspecified, but every memory access stays
 *    inside the buffers the shapes describe.  With value checks on (see
 *    kda_set_validation) they return KDA_ERR_INVALID_VALUE before any work
 *    is launched.  A launch failure reported by the HIP runtime returns
 *    KDA_ERR_HIP.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The stream type of the HIP runtime (same definition as HIP's own header). */
typedef struct ihipStream_t *hipStream_t;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL_ARG = 1,            /* a required pointer is NULL              */
  KDA_ERR_BAD_SHAPE = 2,           /* a size is negative or inconsistent     */
  KDA_ERR_UNSUPPORTED_DIM = 3,     /* d_k or d_v not in {16, 32, 64, 128}    */
  KDA_ERR_UNSUPPORTED_DTYPE = 4,   /* dtype is not KDA_F32 or KDA_BF16        */
  KDA_ERR_MISALIGNED = 5,          /* a tensor pointer is not 16-B aligned   */
  KDA_ERR_WORKSPACE_TOO_SMALL = 6, /* workspace_bytes below the query result */
  KDA_ERR_VARLEN_REQUIRES_B1 = 7,  /* cu_seqlens given with B != 1           */
  KDA_ERR_ALIAS = 8,               /* an output overlaps an input, another
                                      output or the workspace                */
  KDA_ERR_HIP = 9,                 /* the HIP runtime reported an error      */
  KDA_ERR_UNSUPPORTED_GATE = 10,   /* gate is not a kda_gate value           */
  KDA_ERR_INVALID_VALUE = 11,      /* a value check failed (validation on)   */
  KDA_ERR_UNSUPPORTED_ACT = 12,    /* input_act has bits no kda_input_act has */
  KDA_ERR_STREAM_CAPTURE = 13,     /* the call has to wait for the device
                                      (value checks, status query) but the
                                      stream is being captured into a graph  */
  KDA_ERR_TOO_LARGE = 14           /* more scratch than kda_chunk_fwd_noalloc
                                      holds                                  */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/*
 * How the forget gate is given.  Page "Kimi Delta Attention (KDA)": section
 * "KDA: a separate gate for each key channel" gives one gate per key channel;
 * section "Gated DeltaNet: ..." gives one scalar gate per token that scales
 * the whole state; section "DeltaNet: ..." has no gate.  The scalar form is
 * the per-channel form with the same value on every channel, and no gate is
 * the per-channel form with every value 1.
 *   KDA_GATE_CHANNEL      alpha [..., d_k] fp32, one value per key channel
 *   KDA_GATE_SCALAR       alpha [...]      fp32, one value per token and head
 *   KDA_GATE_NONE         no forgetting; alpha is not read and may be NULL
 *   KDA_GATE_LOG_CHANNEL  as KDA_GATE_CHANNEL, holding log(alpha) <= 0
 *   KDA_GATE_LOG_SCALAR   as KDA_GATE_SCALAR, holding log(alpha) <= 0
 *   KDA_GATE_SOFTPLUS_CHANNEL  as KDA_GATE_CHANNEL, holding logits g with
 *                         alpha = exp(-softplus(g)) = 1 / (1 + e^g)
 *   KDA_GATE_SOFTPLUS_SCALAR   the same, one logit per token and head
 * The log forms take the gate as the same page's section "Two schedules of
 * computation for one recurrence" describes the production pipeline taking
 * it (decays as logarithms); a model computing alpha = exp(-softplus(x))
 * passes -softplus(x) and skips the exponential pass over the gates.  The
 * kernels take exp on load (fp32, hardware exp2 of g log2 e, relative error
 * about |g| 2^-23; -inf gives a gate of exactly 0) and
 * then run unchanged.  The softplus forms take the gate of the model code
 * around the method (alpha = exp(-softplus(g)), the gate of the prefill
 * workload's recipe) straight from its logits; large g gives 0.  Gates must lie in [0, 1] (log gates in [-inf, 0]);
 * values outside are not checked and give unspecified results.
 */
typedef enum {
  KDA_GATE_CHANNEL = 0,
  KDA_GATE_SCALAR = 1,
  KDA_GATE_NONE = 2,
  KDA_GATE_LOG_CHANNEL = 3,
  KDA_GATE_LOG_SCALAR = 4,
  KDA_GATE_SOFTPLUS_CHANNEL = 5,
  KDA_GATE_SOFTPLUS_SCALAR = 6
} kda_gate;

/*
 * Activations applied to raw inputs as the kernels load them (bit flags),
 * so a model needs no separate pass over q, k and beta.  They are those of
 * the delta-rule block's model code on the pages (page "22580: from GPT-2
 * to Kimi K3, explained", section "DeltaNet, or Fast Weight Programmers",
 * the forward of the layer with a write strength): q and k
 * go through SiLU and are then scaled to unit length over d_k per token and
 * head (x / max(|x|, 1e-12)); beta goes through a sigmoid.  fp32 math on
 * the hardware exponential, reciprocal and reciprocal square root.
 */
typedef enum {
  KDA_ACT_NONE = 0,
  KDA_ACT_QK_SILU_L2NORM = 1,
  KDA_ACT_BETA_SIGMOID = 2
} kda_input_act;

/* Text for a status code (static storage; never NULL). */
const char *kda_status_string(kda_status s);

/*
 * Value checks, a debugging aid: with enable != 0 every compute entry point
 * first runs a device kernel over its inputs and returns
 * KDA_ERR_INVALID_VALUE, launching nothing else, if
 *   - a gate is outside [0, 1] (a log gate above 0), or NaN,
 *   - a beta is outside [0, 1], or NaN,
 *   - a key's squared norm differs from 1 by more than 1/64 (page "Kimi
 *     Delta Attention (KDA)", section "DeltaNet: writing the error instead of
 *     the value": the write replaces the value stored along k when |k| = 1),
 *   - cu_seqlens does not start at 0, decreases, or does not end at T.
 * The check reads every input once more and then SYNCHRONISES `stream`
 * (with kda_chunk_fwd_status, the only cases in which a call waits for the
 * device), so on a stream being captured into a graph a call with checks on
 * returns KDA_ERR_STREAM_CAPTURE.  Checks from several host threads run one
 * at a time.  The initial state is on when the environment variable
 * KDA_VALIDATE holds a nonzero integer at load time.  Process-wide; returns
 * the previous setting (enable < 0 only returns the current one).
 */
int kda_set_validation(int enable);

/*
 * How kda_chunk_fwd schedules its two kernels (chunk preparation, which is
 * parallel over all chunks, and the scan, which walks each sequence's chunks
 * in order; page "Kimi Delta Attention (KDA)", section "Two schedules of
 * computation for one recurrence").
 *   KDA_SCHEDULE_TWO_PHASE: the preparation of every chunk, then the scan,
 *     on `stream`.
 *   KDA_SCHEDULE_OVERLAP: both at once on two internal streams confined to
 *     disjoint sets of compute units (128 for the scan, 112 for the
 *     preparation), the scan copying each chunk's
 *     record as soon as its preparation is published (ready bits in the
 *     workspace; producer and consumer of a record run on the same XCD, so
 *     the record is read from that XCD's L2).  The call forks from and joins
 *     back to `stream` with events, so it stays asynchronous and ordered on
 *     `stream`.  Used for dense bf16 batches with d_k = d_v = 128 on a full
 *     MI355X (256 CUs); other calls run two-phase, and so does every call
 *     made while `stream` is being captured into a graph (a replay keeps
 *     neither the compute-unit masks nor the concurrency the scan waits
 *     on).  Both schedules give bitwise identical results.  Calls from
 *     several host threads are serialised around the internal streams,
 *     which are created on the first overlapped call on a device (if that
 *     fails, the device stays on two-phase) and released by kda_release().
 *     If the preparation cannot run for more than about a second (another
 *     process holding its compute units), the scan stops waiting and its
 *     results are wrong: kda_chunk_fwd_status then reports
 *     KDA_SCHED_ERR_TIMEOUT for that workspace.
 *   KDA_SCHEDULE_SPLIT: split-sequence, for long sequences over few heads
 *     (page "Kimi Delta Attention (KDA)": the state has a fixed size, which
 *     is what makes very long contexts feasible; the chunk-to-chunk step is
 *     affine in the state).  Each sequence is cut into G segments of whole
 *     chunks.  After the preparation, one pass computes for every segment
 *     but the last the affine map of the state over it (S_end = S_start M +
 *     X: the scan from S = 0 gives X, the scan from the identity with v = 0
 *     gives M), a small pass chains the maps into each segment's start state
 *     (in fp32), and the scan then runs all segments at once.  The result
 *     equals the other schedules' up to rounding (not bitwise: the start
 *     states come from the maps).  Dense bf16 batches with d_k = d_v = 128
 *     whose B * H leaves room for it (G >= 2 segments of at least 16
 *     chunks whose modelled cost beats the sequential scan); other calls run
 *     as under KDA_SCHEDULE_AUTO.  Needs the larger workspace
 *     kda_chunk_fwd_workspace_size reports for those shapes.
 *   KDA_SCHEDULE_AUTO (default): split-sequence when supported and its
 *     modelled cost is at most 3/4 of the sequential scan's (for example
 *     B = 1, H = 8, T = 65536); else overlap when supported, the scan's
 *     workgroups (B * H * d_v / 32) fit on 128 compute units, and the batch
 *     holds at least 4096 chunks over all sequences and heads
 *     (B * H * ceil(T / 64); long sequences over few heads, whose records
 *     overflow the Infinity Cache); else two-phase.
 * The initial value is taken from the environment variable KDA_SCHEDULE
 * (0, 1, 2 or 3) at load time.  Process-wide; returns the previous setting,
 * or -1 (nothing changed) for an unknown value.
 */
typedef enum {
  KDA_SCHEDULE_AUTO = 0,
  KDA_SCHEDULE_TWO_PHASE = 1,
  KDA_SCHEDULE_OVERLAP = 2,
  KDA_SCHEDULE_SPLIT = 3
} kda_schedule;
int kda_set_schedule(int schedule);

/*
 * What the last kda_chunk_fwd call that launched work with this workspace
 * did: *schedule receives the schedule it ran (KDA_SCHEDULE_TWO_PHASE,
 * KDA_SCHEDULE_OVERLAP or KDA_SCHEDULE_SPLIT) and *errors the overlapped schedule's error bits
 * (0 for a clean call; KDA_SCHED_ERR_TIMEOUT: a wait for a chunk record gave
 * up, so that call's o and S_final are wrong; KDA_SCHED_ERR_XCD: a record
 * was read on another XCD than the one that wrote it).  The workspace keeps
 * these words in its first 256 bytes.  Reads them with a copy on `stream`
 * and SYNCHRONISES the stream (so returns KDA_ERR_STREAM_CAPTURE while it
 * is being captured).  Either output pointer may be NULL.  Before any call
 * has used the workspace the words are whatever it held.
 */
enum { KDA_SCHED_ERR_TIMEOUT = 1, KDA_SCHED_ERR_XCD = 2 };
kda_status kda_chunk_fwd_status(const void *workspace, hipStream_t stream,
                                int *schedule, unsigned *errors);

/*
 * Destroys the internal streams and events the overlapped schedule created
 * (after the work queued on them finishes), on every device.  Idempotent;
 * a later overlapped call creates them again.  Also registered with atexit
 * by the first call that creates them.
 */
void kda_release(void);

/*
 * The bound on one wait of the overlapped schedule's scan for a chunk
 * record, in ticks of the GPU's 100 MHz real-time counter (default 2^27,
 * about 1.3 s); a wait that reaches it gives up, so the kernel always ends,
 * and sets KDA_SCHED_ERR_TIMEOUT.  0 gives up at once without waiting: the
 * way to exercise that error path on purpose (the call's results are then
 * wrong).  Process-wide; returns the previous value (ticks < 0 only returns
 * the current one).
 */
long long kda_set_sched_wait_limit(long long ticks);

/*
 * Bytes of device workspace kda_chunk_fwd needs for these sizes (host-only
 * arithmetic, no device call).  For a packed batch pass B = 1 and N = the
 * number of sequences; for a dense batch N may be anything (with B = 1 and
 * N >= 0 the result covers both readings).  Returns 0 for invalid sizes.
 */
size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int d_k, int d_v,
                                    int N, kda_dtype dtype);

/*
 * Chunked prefill over whole sequences (page "Kimi Delta Attention (KDA)",
 * section "Two schedules for one recurrence", the chunkwise schedule).
 *
 *  q, k     [B, T, H, d_k]  dtype      queries, unit-norm keys
 *  v        [B, T, H, d_v]  dtype      values
 *  alpha    [B, T, H, d_k]  fp32       per-key-channel forget gates
 *  beta     [B, T, H]       fp32       write strengths
 *  S0       [N, H, d_v, d_k] fp32      initial states, or NULL for zeros
 *  cu_seqlens [N+1] int32, device, or NULL.  With offsets the batch is a
 *           packed one: B must be 1, T is the packed token count, and
 *           sequence n owns tokens [cu_seqlens[n], cu_seqlens[n+1]) (a
 *           zero-length sequence leaves its state unchanged).  No state flows
 *           between sequences.  Without offsets N is ignored (N = B).
 *  scale    read scale; <= 0 selects d_k^{-1/2}
 *  o        [B, T, H, d_v]  dtype      outputs (must not overlap an input)
 *  S_final  [N, H, d_v, d_k] fp32      final states; may be the same buffer
 *           as S0 (in-place update)
 *  workspace / workspace_bytes: device scratch of at least
 *           kda_chunk_fwd_workspace_size(B, T, H, d_k, d_v, N, dtype) bytes
 *           (at least 256 for any shape), 16-B aligned; its contents on
 *           entry do not matter.  It must not overlap any other argument;
 *           S_final must not overlap an input unless it is exactly S0.
 *
 * T = 0 (or an empty packed batch) copies S0 (or zeros) to S_final.
 * Size limits: B T < 2^31 tokens, and H d_v < 2^23 (64 token rows of every
 * head's outputs in fp32 span less than 2^31 bytes); beyond either the call
 * returns KDA_ERR_BAD_SHAPE and the workspace query returns 0.
 */
kda_status kda_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *alpha, const float *beta,
                         const float *S0, const int32_t *cu_seqlens, int N,
                         int B, int T, int H, int d_k, int d_v, float scale,
                         kda_dtype dtype, void *o, float *S_final,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * kda_chunk_fwd with the gate given as `gate` (see kda_gate): alpha is
 * [B, T, H, d_k] for KDA_GATE_CHANNEL (then this is kda_chunk_fwd) and
 * KDA_GATE_LOG_CHANNEL, [B, T, H] for KDA_GATE_SCALAR and
 * KDA_GATE_LOG_SCALAR, and unused (may be NULL) for KDA_GATE_NONE.
 * Everything else as for kda_chunk_fwd; an unknown gate returns
 * KDA_ERR_UNSUPPORTED_GATE.
 */
kda_status kda_chunk_fwd_gated(const void *q, const void *k, const void *v,
                               const float *alpha, kda_gate gate, const float *beta,
                               const float *S0, const int32_t *cu_seqlens, int N,
                               int B, int T, int H, int d_k, int d_v, float scale,
                               kda_dtype dtype, void *o, float *S_final,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * One decode step for N independent sequences (page "Kimi Delta Attention
 * (KDA)", section "Two schedules for one recurrence", the fused recurrent
 * schedule): every (n, h) state takes one token and is updated in place.
 *
 *  q, k     [N, H, d_k]  dtype     v [N, H, d_v]  dtype
 *  alpha    [N, H, d_k]  fp32      beta [N, H]   fp32
 *  S        [N, H, d_v, d_k] fp32  read and overwritten with the new state
 *  o        [N, H, d_v]  dtype     must not overlap S or an input
 *  scale    <= 0 selects d_k^{-1/2}
 */
kda_status kda_decode_step(const void *q, const void *k, const void *v,
                           const float *alpha, const float *beta, float *S,
                           int N, int H, int d_k, int d_v, float scale,
                           kda_dtype dtype, void *o, hipStream_t stream);

/*
 * kda_decode_step with the gate given as `gate`: alpha is [N, H, d_k] for
 * the per-channel forms, [N, H] for the scalar forms, unused (may be NULL)
 * for KDA_GATE_NONE.  An unknown gate returns KDA_ERR_UNSUPPORTED_GATE.
 */
/*
 * kda_chunk_fwd_gated with input activations: input_act is a bitwise OR of
 * kda_input_act flags, applied to the raw q, k and beta before the method
 * (with KDA_ACT_QK_SILU_L2NORM, k need not be a unit vector).  Unknown bits
 * return KDA_ERR_UNSUPPORTED_ACT.  Everything else as for kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_ex(const void *q, const void *k, const void *v,
                            const float *alpha, kda_gate gate, const float *beta,
                            unsigned input_act, const float *S0,
                            const int32_t *cu_seqlens, int N, int B, int T, int H,
                            int d_k, int d_v, float scale, kda_dtype dtype, void *o,
                            float *S_final, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * The operations around the method in a KDA block, fused into the prefill
 * (page "K3 架构图解": chapter 08, "KDA 与 MLA 如何混合", figure caption:
 * the KDA module holds a short convolution, a normalisation and an output
 * gate besides the recurrence; chapter 09: the short convolution, like the
 * recurrence, depends on token order, so it is causal; chapter 05, section
 * on the extra norm: RMSNorm(u) = gamma * u / sqrt(mean(u^2) + eps);
 * chapter 07: a per-coordinate gate on the concatenated head outputs before
 * the output projection).  Every member is optional (NULL: that operation
 * is not applied).
 *
 *  conv_q, conv_k  [H, d_k, 4] fp32   conv_v  [H, d_v, 4] fp32
 *      Short convolution: all three, or none.  Channel c of head h of q (k,
 *      v) at token t becomes  sum_{i=0..3} w[h][c][i] * x[t-3+i]  over the
 *      token and the three before it in its own sequence (tokens before the
 *      sequence's first count as zero: no convolution state flows in from a
 *      previous call), rounded to dtype.  Requires KDA_ACT_QK_SILU_L2NORM,
 *      which then applies to the convolved q and k; v gets no activation.
 *      Runs the two-phase schedule.
 *  norm_weight  [d_v] fp32, norm_eps
 *      RMS norm of each output row (token, head) over its d_v values, with
 *      gains norm_weight shared by the heads:  o <- o / sqrt(mean(o^2) +
 *      norm_eps) * norm_weight.
 *  out_gate  same layout and dtype as o
 *      Output gate:  o <- o * sigmoid(out_gate)  elementwise (after the norm
 *      when both are given).
 *  conv_state  [N, H, 3, 2 d_k + d_v] dtype: the raw (unconvolved) q, k
 *      and v of three consecutive tokens of each sequence, oldest first,
 *      each token laid out q | k | v.  kda_chunk_fwd_module writes there,
 *      when given, the last three tokens of each sequence (zeros for the
 *      positions before a sequence shorter than three), which is what
 *      kda_decode_tokens_module needs to continue it.  The decode entry point
 *      reads it as the three tokens before its first, and replaces it by the
 *      last three of (those, then its Tk tokens).  Optional for the prefill,
 *      required by the decode entry point with the convolution; must not
 *      overlap any other argument.
 * The norm and gate run in fp32 on the outputs as rounded to dtype, and
 * round once more.  In a packed batch, rows of o outside every sequence are
 * left alone.
 */
typedef struct {
  const float *conv_q, *conv_k, *conv_v;
  const float *norm_weight;
  float norm_eps;
  const void *out_gate;
  void *conv_state;
} kda_module_ops;

/*
 * kda_chunk_fwd_ex with the operations of kda_module_ops (ops may be NULL:
 * then this is kda_chunk_fwd_ex).  Returns KDA_ERR_NULL_ARG when only some
 * of the three convolution weights are given, KDA_ERR_UNSUPPORTED_ACT when
 * they are given without KDA_ACT_QK_SILU_L2NORM, KDA_ERR_MISALIGNED for a
 * weight or gate pointer not 16-byte aligned, KDA_ERR_BAD_SHAPE for a
 * negative or NaN norm_eps, and KDA_ERR_ALIAS when o overlaps a weight or
 * the gate.  Everything else as for kda_chunk_fwd.
 */
kda_status kda_chunk_fwd_module(const void *q, const void *k, const void *v,
                                const float *alpha, kda_gate gate,
                                const float *beta, unsigned input_act,
                                const kda_module_ops *ops, const float *S0,
                                const int32_t *cu_seqlens, int N, int B, int T,
                                int H, int d_k, int d_v, float scale,
                                kda_dtype dtype, void *o, float *S_final,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * kda_chunk_fwd_ex for callers that cannot allocate device memory: code
 * being captured into a HIP graph, tight serving loops, harnesses that
 * forbid allocation.  It takes no workspace: the kernels run on a static
 * device array of the library's own, 64 MiB per device, held until the
 * process ends.  The call itself allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine) and always runs the two-phase
 * schedule; value checks (kda_set_validation) do not apply to it.
 *  - A dense batch whose workspace (kda_chunk_fwd_workspace_size) fits in
 *    64 MiB runs as one call.  A larger dense batch runs one sequence at a
 *    time, in segments of whole 64-token chunks that fit, each segment
 *    starting from the state the previous one left in S_final: the same
 *    chunks and the same arithmetic, so the results equal kda_chunk_fwd_ex's
 *    bit for bit.  Sizes where not even one chunk per head fits return
 *    KDA_ERR_TOO_LARGE.
 *  - A packed batch (cu_seqlens) must fit whole, else KDA_ERR_TOO_LARGE.
 * Every call on a device shares that device's array, which keeps the last
 * call's contents: calls that overlap in time on one device (two streams,
 * or two host threads) race and give wrong results; serialise them.
 */
kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const float *alpha, kda_gate gate,
                                 const float *beta, unsigned input_act,
                                 const float *S0, const int32_t *cu_seqlens,
                                 int N, int B, int T, int H, int d_k, int d_v,
                                 float scale, kda_dtype dtype, void *o,
                                 float *S_final, hipStream_t stream);

/*
 * kda_decode_tokens_ex with the operations of kda_module_ops (ops may be
 * NULL: then this is kda_decode_tokens_ex): the short convolution (its
 * conv_state required: the three raw tokens before the launch's first,
 * replaced by the last three; needs KDA_ACT_QK_SILU_L2NORM), then the output
 * norm and gate on each (token, head) row.  The convolved q, k and v are
 * rounded to dtype, as in kda_chunk_fwd_module, so a prefill followed by
 * decode steps convolves every token as one prefill over all of them would.
 * out_gate is [N, Tk, H, d_v] dtype.  Error returns as for
 * kda_chunk_fwd_module, and KDA_ERR_NULL_ARG for a missing conv_state.
 */
kda_status kda_decode_tokens_module(const void *q, const void *k, const void *v,
                                    const float *alpha, kda_gate gate,
                                    const float *beta, unsigned input_act,
                                    const kda_module_ops *ops,
                                    const float *S_in, float *S_out, int N,
                                    int Tk, int H, int d_k, int d_v, float scale,
                                    kda_dtype dtype, void *o, hipStream_t stream);

kda_status kda_decode_step_gated(const void *q, const void *k, const void *v,
                                 const float *alpha, kda_gate gate,
                                 const float *beta, float *S, int N, int H,
                                 int d_k, int d_v, float scale, kda_dtype dtype,
                                 void *o, hipStream_t stream);

/*
 * Several tokens per sequence in one launch, taken in order by the
 * token-by-token schedule, for verifying a draft of speculative decoding
 * (page "K3 架构图解", chapter 10: a draft model proposes tokens, the target
 * model verifies them together, and the recurrent state has to be kept
 * where a rejected token can be undone).  Each (n, h) state is read from
 * S_in once, carried through its Tk tokens in registers, and written to
 * S_out once.  With S_out a different buffer, S_in stays the checkpoint to
 * roll back to (run again on the accepted prefix); S_out == S_in updates in
 * place.  Tk = 0 copies S_in to S_out.
 *
 *  q, k     [N, Tk, H, d_k]  dtype     v [N, Tk, H, d_v]  dtype
 *  alpha    [N, Tk, H, d_k] (per-channel forms), [N, Tk, H] (scalar
 *           forms), unused (KDA_GATE_NONE)    beta [N, Tk, H]  fp32
 *  S_in, S_out [N, H, d_v, d_k] fp32: the same buffer or disjoint ones
 *           (a partial overlap returns KDA_ERR_ALIAS)
 *  o        [N, Tk, H, d_v]  dtype     must not overlap an input or a state
 *  scale    <= 0 selects d_k^{-1/2}
 */
kda_status kda_decode_tokens(const void *q, const void *k, const void *v,
                             const float *alpha, kda_gate gate,
                             const float *beta, const float *S_in,
                             float *S_out, int N, int Tk, int H, int d_k,
                             int d_v, float scale, kda_dtype dtype, void *o,
                             hipStream_t stream);

/*
 * kda_decode_tokens with input activations (see kda_chunk_fwd_ex); with
 * Tk = 1 and S_out == S_in it is a decode step on raw inputs.
 */
kda_status kda_decode_tokens_ex(const void *q, const void *k, const void *v,
                                const float *alpha, kda_gate gate,
                                const float *beta, unsigned input_act,
                                const float *S_in, float *S_out, int N,
                                int Tk, int H, int d_k, int d_v, float scale,
                                kda_dtype dtype, void *o, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
