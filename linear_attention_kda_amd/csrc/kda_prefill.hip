// kda_prefill.hip -- chunkwise KDA prefill for gfx950.
//
// Method: page "Kimi Delta Attention (KDA)" (brain.bigb.es), section "Two
// schedules for one recurrence".  For a chunk of C = 64 tokens starting from
// state S (d_v x d_k), with D_{a:b} the product of the gates alpha_a..alpha_b
// (empty product = identity; a token's own gate acts before its write):
//
//   provisional errors  ebar_i = beta_i (v_i - S D_{0:i} k_i)
//   coupling            rho_ij = beta_i k_j^T D_{j+1:i} k_i      (j < i)
//   true errors         E = (I + R)^{-1} Ebar       (rows e_i, causal solve)
//   next state          S' = S D_{0:63} + E^T Kend,  Kend_j = D_{j+1:63} k_j
//   outputs             O = s Qbnd S^T + A E,  A_ij = s k_j^T D_{j+1:i} q_i
//                       (j <= i: a token reads its own write)
//
// Split used here (E = T Diag(beta) (V - Kbnd S^T) with T = (I + R)^{-1}):
//
//   kernel 1 (chunk prep, one workgroup per (chunk, head), fully parallel):
//     products of the gates per key channel -> Kbnd = k*D_{0:i},
//     Qbnd = q*D_{0:i}, Kend (transposed) and D_{0:63}; A^kk and A^qk on the
//     matrix cores, factorised per 16-token block pair; R -> T by blocked
//     forward substitution (16x16 diagonal blocks inverted on the vector
//     ALUs, off-diagonal blocks by fp32 MFMA); writes Tb = T Diag(beta) and A
//     to a per-chunk workspace record.
//   kernel 2 (scan, one compute wave per (sequence, head, 16 value columns),
//     fed by a copy wave that streams chunk records into LDS): walks the
//     chunks in order with S^T held in MFMA accumulators (fp32):
//     X = [Kbnd; Qbnd] S^T, Ebar = V - X_top, E = Tb Ebar,
//     O = s X_bot + A E, S^T = D_{0:63} S^T + Kend^T E.
//
// A^kk and A^qk are built per 16-token block pair from products of the gates
// (see chunk_prep_kernel); no step divides by a decay that can underflow, so
// gates of any strength in [0, 1], including exact zeros, are handled.
#include "kda_device.h"
#include "kda_launch.h"

#include <hip/hip_ext.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

namespace kda {
namespace {

// ============================================================ index kernel
// Packed batch -> monotone clamped sequence offsets, chunk counts and the
// chunk list.  Offsets are clamped to [0, T] and made non-decreasing, so every
// token index used later stays inside the buffers even for malformed input.
__global__ __launch_bounds__(1024) void varlen_index_kernel(
    const int32_t *__restrict__ cu, int N, int T, int32_t *seq_tok0,
    int32_t *seq_chunk0, int32_t *chunk_t0, int32_t *chunk_len, int32_t *chunk_s0,
    long long max_chunks, int32_t *seq_order) {
  __shared__ int32_t s[1024];
  const int tid = threadIdx.x;
  int tok_carry = 0;    // offset of the entry before this tile
  int chunk_carry = 0;  // chunks of all sequences before this tile's first
  for (int base = 0; base <= N; base += 1024) {
    const int n = base + tid;
    int x = 0;
    if (n <= N) {
      x = cu[n];
      x = x < 0 ? 0 : (x > T ? T : x);
    }
    x = max(x, tok_carry);
    s[tid] = x;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int y = tid >= off ? s[tid - off] : 0;
      __syncthreads();
      if (tid >= off) s[tid] = max(s[tid], y);
      __syncthreads();
    }
    const int e = s[tid];
    const int e_prev = tid > 0 ? s[tid - 1] : tok_carry;
    const int next_tok_carry = s[1023];
    if (n <= N) seq_tok0[n] = e;
    const int m = n - 1;  // sequence m spans [e_prev, e)
    int cnt = 0;
    if (m >= 0 && m < N) cnt = (e - e_prev + kChunk - 1) / kChunk;
    __syncthreads();
    s[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int y = tid >= off ? s[tid - off] : 0;
      __syncthreads();
      if (tid >= off) s[tid] += y;
      __syncthreads();
    }
    const int excl = s[tid] - cnt + chunk_carry;
    const int next_chunk_carry = s[1023] + chunk_carry;
    if (m >= 0 && m < N) {
      seq_chunk0[m] = excl;
      for (int j = 0; j < cnt; ++j) {
        long long c = (long long)excl + j;
        if (c < max_chunks) {
          chunk_t0[c] = e_prev + kChunk * j;
          chunk_len[c] = min(kChunk, e - e_prev - kChunk * j);
          chunk_s0[c] = e_prev;  // the sequence's first token
        }
      }
    }
    tok_carry = next_tok_carry;
    chunk_carry = next_chunk_carry;
    __syncthreads();
  }
  if (tid == 0) seq_chunk0[N] = chunk_carry;

  // Scan order, longest sequence first: the scan's sequential chain of a
  // sequence is as long as its chunk count, and the longest chains should
  // not start last.  seq_order[r] is the sequence of rank r (more chunks
  // first, ties by index), from a rank count over all pairs in LDS; with
  // more than 1024 sequences the order stays the identity.
  __syncthreads();  // seq_chunk0 complete (written by this workgroup)
  if (N <= 1024) {
    const int cnt = tid < N ? seq_chunk0[tid + 1] - seq_chunk0[tid] : -1;
    s[tid] = cnt;
    __syncthreads();
    if (tid < N) {
      int r = 0;
      for (int j = 0; j < N; ++j) r += s[j] > cnt || (s[j] == cnt && j < tid);
      seq_order[r] = tid;
    }
  } else {
    for (int i = tid; i < N; i += 1024) seq_order[i] = i;
  }
}

struct ChunkSource {
  // dense batch: sequence n starts at token n*T, nct chunks per sequence
  int T, nct;
  // packed batch (device tables; null for dense)
  const int32_t *chunk_t0, *chunk_len, *chunk_s0, *seq_chunk0;
  int n_seq;
};

// Chunk slot c: its first token t0, its length L and the first token s0 of
// its sequence; false for a slot past the last chunk.
__device__ __forceinline__ bool chunk_span(const ChunkSource &cs, long long c,
                                           long long &t0, int &L, long long &s0) {
  if (cs.chunk_t0) {
    if (c >= cs.seq_chunk0[cs.n_seq]) return false;
    t0 = cs.chunk_t0[c];
    L = cs.chunk_len[c];
    s0 = cs.chunk_s0[c];
  } else {
    const long long n = c / cs.nct, ci = c % cs.nct;
    s0 = n * cs.T;
    t0 = s0 + ci * kChunk;
    L = (int)min((long long)kChunk, (long long)cs.T - ci * kChunk);
  }
  return true;
}

// ======================================================= fragment order
// A operands of the 16x16 products are stored so that each lane's share of a
// (16-row tile, k-slab) fragment is contiguous.  bf16 with K % 32 == 0 uses
// v_mfma_f32_16x16x32_bf16 slabs of 32 columns: lane (row r, group g) holds
// columns 4g..4g+3 then 16+4g..16+4g+3 of the slab (8 elements, 16 bytes).
// bf16 with K == 16 and fp32 use slabs of 16 columns: lane (r, g) holds columns
// 4g..4g+3 (bf16: 8 bytes for 16x16x16; fp32: 16 bytes, four 16x16x4 steps).
// The B operands that meet these fragments come from accumulator tiles, whose
// lane (column, g) holds rows 4g..4g+3, so the k order matches with no shuffle.
template <typename E, int K> struct FragShape {
  static constexpr bool wide = sizeof(E) == 2 && K % 32 == 0;
  static constexpr int W = wide ? 32 : 16;  // columns per slab
  static constexpr int KS = W / 4;          // elements per lane per fragment
  static constexpr int NU = K / W;          // slabs per 16-row tile
};

// Element offset of A(i, c) in fragment order.
template <typename E, int K>
__device__ __forceinline__ int frag_index(int i, int c) {
  typedef FragShape<E, K> F;
  const int ci = c % F::W;
  int g, pos;
  if constexpr (F::wide) {
    const int cc = ci & 15;
    g = cc >> 2;
    pos = (ci >> 4) * 4 + (cc & 3);
  } else {
    g = ci >> 2;
    pos = ci & 3;
  }
  return (((i >> 4) * F::NU + c / F::W) * 64 + (i & 15) + 16 * g) * F::KS + pos;
}

// Element offset of A(i, c) in a lower-triangular 64 x 64 operand stored
// without its zero slabs (tri_slab0 in kda_launch.h); the position rule within
// a fragment is that of frag_index.
template <typename E>
__device__ __forceinline__ int tri_index(int i, int c) {
  typedef FragShape<E, 64> F;
  const int ci = c % F::W;
  int g, pos;
  if constexpr (F::wide) {
    const int cc = ci & 15;
    g = cc >> 2;
    pos = (ci >> 4) * 4 + (cc & 3);
  } else {
    g = ci >> 2;
    pos = ci & 3;
  }
  return ((tri_slab0(i >> 4, (int)sizeof(E)) + c / F::W) * 64 + (i & 15) + 16 * g) * F::KS + pos;
}

// ======================================================= kernel 1: chunk prep
struct PrepKArgs {
  const void *q, *k;
  const float *alpha, *beta;
  int gate;  // a kGate* form: alpha [.., H, d_k] per channel, [.., H] per token, unused for none
  unsigned act;  // kAct* input activations
  ChunkSource src;
  int H;
  float scale;
  char *ws_records;
  ChunkRecordLayout lay;
  // overlapped schedule (null otherwise): the ready words (ready_words per
  // unit), the control words (kCtlWords) and the number of units
  int *ready, *ctl;
  int ready_words, n_units;
  // short convolution (CONV instantiations only): taps [H, d, kConvTaps] of
  // q, k and v; v [.., H, dv] is read and its convolution written to o
  const float *conv_q, *conv_k, *conv_v;
  const void *v;
  void *o;
  int dv;
};

// Index of the XCD (accelerator complex die) this wave runs on, 0..7.  Each
// XCD has its own L2; the overlapped schedule keeps the producer and the
// consumer of every chunk record on one XCD.
__device__ __forceinline__ int xcd_id() {
  unsigned x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return (int)(x & 7);
}

// LDS image of a fragment-ordered operand (FragShape<E, K>, ROWS rows), slot
// by slot in record order.  Within each 16-row group the rows are XOR-swizzled
// by (g + 4 (slab & 1)) & 7, so that both a wave writing four channels of one
// row per lane and a wave reading one 16-byte slot per lane spread over all
// LDS banks.
template <typename E, int K, int ROWS> struct LdsFrag {
  typedef FragShape<E, K> F;
  static constexpr int SLOT = F::KS * (int)sizeof(E);  // bytes per lane slot (16 or 8)
  static constexpr int NSLOT = ROWS / 16 * F::NU * 64;
  static constexpr int BYTES = NSLOT * SLOT;
  __device__ __forceinline__ static int slot_off(int tile, int slab, int row16, int g) {
    const int sw = (g + 4 * (slab & 1)) & 7;
    return (((tile * F::NU + slab) * 4 + g) * 16 + (row16 ^ sw)) * SLOT;
  }
  // byte offset of element (row, col); col % 4 == 0 starts 4 contiguous elements
  __device__ __forceinline__ static int elem_off(int row, int col) {
    const int ci = col % F::W;
    int g, pos;
    if constexpr (F::wide) {
      g = (ci & 15) >> 2;
      pos = (ci >> 4) * 4 + (ci & 3);
    } else {
      g = ci >> 2;
      pos = ci & 3;
    }
    return slot_off(row >> 4, col / F::W, row & 15, g) + pos * (int)sizeof(E);
  }
  // LDS byte offset of record slot s = (tile NU + slab) 64 + row16 + 16 g
  __device__ __forceinline__ static int rec_slot(int s) {
    const int ts = s >> 6, L = s & 63;
    return slot_off(ts / F::NU, ts % F::NU, L & 15, L >> 4);
  }
};

template <int BYTES> struct VecOf;
template <> struct VecOf<16> { typedef f32x4 type; };
template <> struct VecOf<8> { typedef __attribute__((__vector_size__(8))) float type; };

// LDS image -> record (global), one slot per thread per step, coalesced.
// Threads t0 .. t0 + nthr - 1 of the workgroup take part.
template <typename LF>
__device__ __forceinline__ void copy_out(char *dst, const char *lds, int t0 = 0, int nthr = kThreads) {
  typedef typename VecOf<LF::SLOT>::type V;
  if ((int)threadIdx.x < t0) return;
  for (int s = threadIdx.x - t0; s < LF::NSLOT; s += nthr)
    *reinterpret_cast<V *>(dst + (size_t)s * LF::SLOT) = *reinterpret_cast<const V *>(lds + LF::rec_slot(s));
}

// Column of element e (0 .. KS-1) of the slot (slab, g) of FragShape<E, K>;
// the inverse of the position rule in frag_index.
template <typename E, int K>
__device__ __forceinline__ int slot_col(int slab, int g, int e) {
  typedef FragShape<E, K> F;
  if constexpr (F::wide) return slab * F::W + (e >> 2) * 16 + 4 * g + (e & 3);
  else return slab * F::W + 4 * g + e;
}

// One record slot (KS elements of E) packed from fp32.
template <typename E, int KS> struct SlotVec;
template <> struct SlotVec<bf16, 8> {
  typedef bf16x8 type;
  __device__ __forceinline__ static type pack(const float *x) {
    type v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
    return v;
  }
};
template <> struct SlotVec<float, 4> {
  typedef f32x4 type;
  __device__ __forceinline__ static type pack(const float *x) { return f32x4{x[0], x[1], x[2], x[3]}; }
};

// Row tiles I0 .. I1-1 of a 64 x 64 fp32 tile in LDS (row stride LDR), masked
// to j <= i and scaled per column by colscale (or not), to a lower-triangular
// record operand (tri_index layout), slot by slot, by threads t0 .. t0 + nthr - 1.
template <typename E, int LDR>
__device__ __forceinline__ void tile64_out(E *dst, const float *src, const float *colscale, int I0 = 0, int I1 = 4,
                                           int t0 = 0, int nthr = kThreads) {
  typedef FragShape<E, 64> F;
  typedef SlotVec<E, F::KS> SV;
  constexpr int es = (int)sizeof(E);
  if ((int)threadIdx.x < t0) return;
  for (int s = tri_slab0(I0, es) * 64 + threadIdx.x - t0; s < tri_slab0(I1, es) * 64; s += nthr) {
    const int fr = s >> 6, L = s & 63;
    int I = 0;
#pragma unroll
    for (int J = 1; J < 4; ++J) I += fr >= tri_slab0(J, es);
    const int i = 16 * I + (L & 15), slab = fr - tri_slab0(I, es), g = L >> 4;
    float x[F::KS];
#pragma unroll
    for (int e = 0; e < F::KS; ++e) {
      const int j = slot_col<E, 64>(slab, g, e);
      x[e] = j <= i ? src[i * LDR + j] * (colscale ? colscale[j] : 1.f) : 0.f;
    }
    *reinterpret_cast<typename SV::type *>(dst + (size_t)s * F::KS) = SV::pack(x);
  }
}

// The gate a stored value stands for, per gate form.
template <int GATE> __device__ __forceinline__ float gate_value(float x) {
  if constexpr (gate_is_log(GATE)) return gate_from_log(x);
  else if constexpr (gate_is_softplus(GATE)) return gate_from_softplus_logit(x);
  else return x;
}

// Sixteen bytes of E as one vector.
template <typename E> struct Row16;
template <> struct Row16<bf16> {
  typedef bf16x8 vec;
  static constexpr int N = 8;
};
template <> struct Row16<float> {
  typedef f32x4 vec;
  static constexpr int N = 4;
};

// Four elements of E from / to fp32.
template <typename E> struct Four;
template <> struct Four<bf16> {
  typedef bf16x4 vec;
  __device__ __forceinline__ static void load(const bf16 *p, float *x) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (float)v[j];
  }
  __device__ __forceinline__ static vec pack(const float *x) {
    vec v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (bf16)x[j];
    return v;
  }
};
template <> struct Four<float> {
  typedef f32x4 vec;
  __device__ __forceinline__ static void load(const float *p, float *x) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = v[j];
  }
  __device__ __forceinline__ static vec pack(const float *x) { return f32x4{x[0], x[1], x[2], x[3]}; }
};

// acc += A_slot * B_slot over one slab (slots read from LDS at byte offsets).
template <typename E, int K>
__device__ __forceinline__ f32x4 slot_mma(const char *pa, const char *pb, f32x4 acc) {
  typedef FragShape<E, K> F;
  if constexpr (sizeof(E) == 4) {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(pa), y = *reinterpret_cast<const f32x4 *>(pb);
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], y[s], acc, 0, 0, 0);
  } else if constexpr (F::wide) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8 *>(pa),
                                                  *reinterpret_cast<const bf16x8 *>(pb), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*reinterpret_cast<const bf16x4 *>(pa),
                                                    *reinterpret_cast<const bf16x4 *>(pb), acc, 0, 0, 0);
  }
  return acc;
}

// Off-diagonal block (I, J), I > J, of T = (I + R)^{-1}:
//   T_IJ = -T_II * sum_{K=J}^{I-1} R_IK T_KJ      (16x16 fp32 blocks, one wave)
template <int LDR>
__device__ __forceinline__ void inverse_offdiag_block(int I, int J, const float *sR, float *sT) {
  const int l = lane_id(), col = l & 15, g = l >> 4;
  f32x4 y = zero4();
  for (int K = J; K < I; ++K) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      y = __builtin_amdgcn_mfma_f32_16x16x4f32(sR[(16 * I + col) * LDR + 16 * K + 4 * s + g],
                                               sT[(16 * K + 4 * s + g) * LDR + 16 * J + col], y, 0, 0, 0);
  }
  // y holds Y[4g + r][col]; feed it back as the B operand with k-slot
  // (g, step s) <-> row 4g + s, matching A = T_II[row][4g + s].
  f32x4 t = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s)
    t = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[(16 * I + col) * LDR + 16 * I + 4 * g + s], y[s], t, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * g + r) * LDR + 16 * J + col] = -t[r];
}

// pair p in 0..9 -> (I, J) of the lower block triangle, row-major
__device__ __forceinline__ void tile_ij(int p, int &I, int &J) {
  I = p >= 6 ? 3 : (p >= 3 ? 2 : (p >= 1 ? 1 : 0));
  J = p - I * (I + 1) / 2;
}

// Chunk prep: one workgroup per (chunk, head); wave b owns the 16-token block
// b, lane (cg, th) owns channels 4cg..4cg+3 for TPL consecutive tokens.
//
// Fast path.  With a_i = D_{0:i} (per channel, products of the gates from the
// chunk start to token i inclusive) every decay between tokens of the chunk
// factors as D_{j+1:i} = a_i / a_j, so
//   R^T = (k / a) (k a)^T,  A^T = (k / a) (s q a)^T   (then masked, R scaled by beta_i)
//   Kbnd = k a,  s Qbnd = s q a,  Kend_j = k_j D_{j+1:63} = (k_j / a_j) D_{0:63}
// are plain products on the matrix cores.  Every a_j >= D_{0:63}, so while
// D_{0:63} >= 2^-100 on every channel no factor exceeds 2^100 and nothing
// over- or underflows in fp32 or bf16.
// Exact path (a chunk with some D_{0:63} below 2^-100, e.g. a gate of 0):
// no division at all.  Kbnd and Qbnd as above, Kend from suffix products, and
// R and A summed channel by channel with running products of the gates.
//
// CONV (with ACTQK, two-phase schedule only): q, k and v first go through a
// depthwise causal convolution over the token and the three before it, within
// the sequence (tokens before its first count as zero), each result rounded
// to E.  q and k are convolved as they are loaded (the three tokens before
// the chunk are read from the previous chunk's rows of the raw input); v's
// convolution is written to o, from where the scan reads it in place of v
// (the scan reads the rows of a chunk before it writes that chunk's outputs
// over them).
template <int DK, typename E, int GATE, bool ACTQK, bool SCHED, bool CONV>
__device__ __forceinline__ void chunk_prep_body(const PrepKArgs &a) {
  typedef LdsFrag<E, DK, 64> LK;   // Kbnd, Qbnd, k / a: rows = tokens, K = d_k
  typedef LdsFrag<E, 64, DK> LT;   // Kend^T: rows = channels, K = tokens
  typedef Four<E> F4;
  constexpr int CG = DK / 4;       // channel groups of four per token
  constexpr int TH = 64 / CG;      // lanes per channel group (token sub-ranges of a block)
  constexpr int TPL = 16 / TH;     // tokens per lane
  constexpr int LDR = 68;          // row stride of the fp32 64x64 tiles
  constexpr int RT_BYTES = 64 * LDR * 4;
  constexpr int SA_BYTES = LT::BYTES > RT_BYTES ? LT::BYTES : RT_BYTES;
  constexpr int P1 = 3 * LK::BYTES;                 // Kbnd | Qbnd | k / a
  constexpr int P2 = 2 * RT_BYTES + SA_BYTES;       // R | T | Kend^T staging or A (exact)
  constexpr int ARENA = P1 > P2 ? P1 : P2;
  static_assert(ARENA >= 4 * DK * 4, "the gate totals live at the start of the arena");
  __shared__ __attribute__((aligned(16))) char arena[ARENA];
  __shared__ float sBeta[kChunk];
  __shared__ float sInvNorm[2][kChunk];  // 1/|SiLU(k)|, 1/|SiLU(q)| per token (input activation only)
  __shared__ float sDiag[kChunk];        // s k_i . q_i per token (the diagonal of A, fast path)

  static_assert(!CONV || (ACTQK && !SCHED), "the convolution comes with the q, k activation, two-phase");
  // one record: chunk slot c, head h
  auto prep_one = [&](const long long c, const int h) {
    long long t0, s0;
    int L;
    if (!chunk_span(a.src, c, t0, L, s0)) return;

    char *rec = a.ws_records + ((size_t)c * a.H + h) * a.lay.bytes;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const int cg = l % CG, th = l / CG, c0 = 4 * cg;
    const E *q = reinterpret_cast<const E *>(a.q);
    const E *k = reinterpret_cast<const E *>(a.k);
    const size_t hs = (size_t)a.H * DK;  // token stride of q, k, alpha
    const size_t base = (size_t)t0 * hs + (size_t)h * DK + c0;
    // gates of channels ch0 .. ch0+3 of token t0 + tk (tk a valid chunk index):
    // per channel, one shared value, or none, given as gates or as their
    // logarithms (see kda_gate)
    // (raw = true: the stored values, for gate_value<GATE> later)
    auto gate4 = [&](int tk, int ch0, float *al, bool nontemporal, bool raw = false) {
      const size_t tok = (size_t)t0 + tk;
      if constexpr (gate_per_channel(GATE)) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(a.alpha + tok * hs + (size_t)h * DK + ch0);
        const f32x4 x = nontemporal ? __builtin_nontemporal_load(p) : *p;
#pragma unroll
        for (int j = 0; j < 4; ++j) al[j] = raw ? x[j] : gate_value<GATE>(x[j]);
      } else {
        float x = 1.f;
        if constexpr (gate_per_token(GATE)) {
          x = a.alpha[tok * a.H + h];
          if (!raw) x = gate_value<GATE>(x);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) al[j] = x;
      }
    };
    const int tb0 = 16 * w + TPL * th;   // first token of this lane
    // CONV: four channels ch.. of token `rel` of the chunk (rel <= L - 1,
    // may be negative) after the convolution, rounded to E
    auto conv_load4 = [&](const E *x, const float *w, int rel, int ch, float *out) {
      f32x4 wt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wt[j] = *reinterpret_cast<const f32x4 *>(w + ((size_t)h * DK + ch + j) * kConvTaps);
      float xs[kConvTaps][4];
#pragma unroll
      for (int i = 0; i < kConvTaps; ++i) {
        const int r = rel - (kConvTaps - 1) + i;
        const bool ok = t0 + r >= s0;
        F4::load(x + (size_t)(t0 + (ok ? r : 0)) * hs + (size_t)h * DK + ch, xs[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) xs[i][j] = ok ? xs[i][j] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) out[j] = (float)(E)conv_taps(wt[j], xs[0][j], xs[1][j], xs[2][j], xs[3][j]);
    };
    // CONV: this lane's TPL tokens (channels c0..c0+3) after the convolution,
    // from the TPL + 3 rows ending at its last token, packed in E
    auto conv_lane = [&](const E *x, const float *w, typename F4::vec *out) {
      constexpr int NW = TPL + kConvTaps - 1;
      typename F4::vec win[NW];
      unsigned okm = 0;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        const int rel = min(tb0 - (kConvTaps - 1) + i, L - 1);
        const bool ok = t0 + rel >= s0;
        okm |= (unsigned)ok << i;
        win[i] = __builtin_nontemporal_load(reinterpret_cast<const typename F4::vec *>(
            x + (size_t)(t0 + (ok ? rel : 0)) * hs + (size_t)h * DK + c0));
      }
      f32x4 wt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) wt[j] = *reinterpret_cast<const f32x4 *>(w + ((size_t)h * DK + c0 + j) * kConvTaps);
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float xv[kConvTaps];
#pragma unroll
          for (int i = 0; i < kConvTaps; ++i) xv[i] = (okm >> (u + i)) & 1 ? (float)win[u + i][j] : 0.f;
          y[j] = conv_taps(wt[j], xv[0], xv[1], xv[2], xv[3]);
        }
        out[u] = F4::pack(y);
      }
    };
    char *sKh = arena, *sQh = arena + LK::BYTES, *sKd = arena + 2 * LK::BYTES;
    float *sR = reinterpret_cast<float *>(arena);
    float *sT = reinterpret_cast<float *>(arena + RT_BYTES);
    char *sX = arena + 2 * RT_BYTES;     // Kend^T staging (fast) or A in fp32 (exact)
    // whole-block gate products; read before the barrier that precedes the
    // first write of the operand images, which reuse this space
    float *sTau = reinterpret_cast<float *>(arena);

    // beta of token tid % 64 (a valid token for every lane: no branch around
    // the load), requested with the inputs below and stored to LDS after them,
    // so no load waits for another
    const float braw = a.beta[(size_t)(t0 + min(tid % kChunk, L - 1)) * a.H + h];

    // ---- loads and in-block prefix products.  Padded tokens (index >= L)
    // take q = k = 0 and alpha = 1; their loads read a valid token instead.
    // Each input byte is read once here, so the loads carry the nontemporal
    // hint (measured faster: they do not displace the records in the caches).
    // q and k stay packed in their own type until used (register budget)
    typename F4::vec kraw[TPL], qraw[TPL];
    float pa[TPL][4];
    if constexpr (CONV) {
      conv_lane(k, a.conv_k, kraw);
      __builtin_amdgcn_sched_barrier(0);  // one tensor's window at a time
      conv_lane(q, a.conv_q, qraw);
    }
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      const int tok = tb0 + u;
      const size_t off = base + (size_t)min(tok, L - 1) * hs;
      float al[4];
      gate4(min(tok, L - 1), c0, al, true, true);   // converted below, after the q, k activation
      if constexpr (!CONV) {
        kraw[u] = __builtin_nontemporal_load(reinterpret_cast<const typename F4::vec *>(k + off));
        qraw[u] = __builtin_nontemporal_load(reinterpret_cast<const typename F4::vec *>(q + off));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) pa[u][j] = al[j];
    }
    if (tid < kChunk) sBeta[tid] = tid < L ? ((a.act & kActBeta) ? sigmoid_f(braw) : braw) : 0.f;
    // k (or q) of token u, channel j, zero for padded tokens
    auto kval = [&](int u, int j) {
      const float x = (float)kraw[u][j];
      return tb0 + u < L ? x : 0.f;
    };
    auto qval = [&](int u, int j) {
      const float x = (float)qraw[u][j];
      return tb0 + u < L ? x : 0.f;
    };
    float tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float run = 1.f;
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        run *= tb0 + u < L ? gate_value<GATE>(pa[u][j]) : 1.f;
        pa[u][j] = run;
      }
      tot[j] = run;
      if constexpr (gate_is_softplus(GATE)) __builtin_amdgcn_sched_barrier(0);
    }
    // exclusive product over the lanes of earlier sub-ranges of the block
    // (lanes cg + CG th' for th' < th); Hillis-Steele scan with stride CG
    float incl[4], excl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) incl[j] = tot[j];
#pragma unroll
    for (int d = 1; d < TH; d <<= 1) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = __shfl(incl[j], l - d * CG);
        if (th >= d) incl[j] *= y;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float y = __shfl(incl[j], l - CG);
      excl[j] = th >= 1 ? y : 1.f;
    }
#pragma unroll
    for (int u = 0; u < TPL; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) pa[u][j] *= excl[j];
    // optional input activation: q, k <- SiLU, then unit length over the d_k
    // channels of the token (CG lanes hold one token's channels)
    if constexpr (ACTQK) {
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        float kx[4], qx[4], sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kx[j] = silu_f((float)kraw[u][j]);
          qx[j] = silu_f((float)qraw[u][j]);
          sk += kx[j] * kx[j];
          sq += qx[j] * qx[j];
        }
        const float rk = inv_norm(group_sum<CG>(sk)), rq = inv_norm(group_sum<CG>(sq));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kx[j] *= rk;
          qx[j] *= rq;
        }
        kraw[u] = F4::pack(kx);
        qraw[u] = F4::pack(qx);
        // the diagonal of A (see below) for a partial chunk, from the
        // values as packed, here where few values are live
        float kq = 0.f;
        if (L < kChunk) {
#pragma unroll
          for (int j = 0; j < 4; ++j) kq = fmaf((float)kraw[u][j], (float)qraw[u][j], kq);
          kq = group_sum<CG>(kq);
        }
        // for the exact path, which reads q and k again from memory
        if (cg == 0) {
          sInvNorm[0][tb0 + u] = rk;
          sInvNorm[1][tb0 + u] = rq;
          sDiag[tb0 + u] = tb0 + u < L ? kq * a.scale : 0.f;
        }
        __builtin_amdgcn_sched_barrier(0);  // one token at a time: bounds the live values
      }
    }
    if (th == TH - 1) *reinterpret_cast<f32x4 *>(sTau + w * DK + c0) = f32x4{incl[0], incl[1], incl[2], incl[3]};
    __syncthreads();

    // ---- chunk prefix a = (blocks before) * (in-block prefix); D_{0:63}
    float fb[4], gb[4], p63[4];
    {
      f32x4 tau[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) tau[b] = *reinterpret_cast<const f32x4 *>(sTau + b * DK + c0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float before = 1.f, after = 1.f;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (b < w) before *= tau[b][j];
          if (b > w) after *= tau[b][j];
        }
        fb[j] = before;
        gb[j] = after;
        p63[j] = tau[0][j] * tau[1][j] * tau[2][j] * tau[3][j];
      }
    }
    int weak = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) weak |= !(p63[j] >= 0x1p-100f);
    const bool exact = __syncthreads_or(weak) != 0;   // uniform over the workgroup

    // ---- Kbnd, s Qbnd (both paths) and k / a (fast path) into LDS
    typename F4::vec ktt[TPL];   // Kend rows of this lane's tokens, packed (written later)
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
      const int tok = tb0 + u;
      float kh[4], qh[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float av = pa[u][j] * fb[j];
        kh[j] = kval(u, j) * av;
        qh[j] = qval(u, j) * av * a.scale;
        pa[u][j] = av;
      }
      *reinterpret_cast<typename F4::vec *>(sKh + LK::elem_off(tok, c0)) = F4::pack(kh);
      *reinterpret_cast<typename F4::vec *>(sQh + LK::elem_off(tok, c0)) = F4::pack(qh);
    }
    // A partial chunk (the end of a sequence; all of a short one) also gets
    // the diagonal of A, s k_i . q_i, summed in fp32 from the values as the
    // kernel holds them (its decays cancel).  The fast path's products take
    // k / a and s q a rounded to E, whose rounding errors do not cancel when
    // k_i . q_i does: a one-token sequence's output is that one term times
    // beta v, so its relative error would be the dot product's condition
    // number times the rounding.  In a full chunk each output row sums up to
    // 64 such terms and the errors average out; there the products' diagonal
    // stands (the sums cost about 1 % of the prefill workload's time).
    const bool diag_exact = L < kChunk;  // uniform over the workgroup
    if constexpr (!ACTQK) {  // (with the activation: summed as q and k are activated)
      if (diag_exact) {
#pragma unroll
        for (int u = 0; u < TPL; ++u) {
          float kq = kval(u, 0) * qval(u, 0);
#pragma unroll
          for (int j = 1; j < 4; ++j) kq = fmaf(kval(u, j), qval(u, j), kq);
          kq = group_sum<CG>(kq);
          if (cg == 0) sDiag[tb0 + u] = kq * a.scale;
        }
      }
    }
    if (!exact) {
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        const int tok = tb0 + u;
        float kd[4], kt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kd[j] = kval(u, j) * __builtin_amdgcn_rcpf(pa[u][j]);
          kt[j] = kd[j] * p63[j];
        }
        *reinterpret_cast<typename F4::vec *>(sKd + LK::elem_off(tok, c0)) = F4::pack(kd);
        ktt[u] = F4::pack(kt);
      }
    } else {
      // D_{j+1:63} without division: in-lane exclusive suffix, times the later
      // sub-ranges of the block, times the later blocks.  The gates are read
      // again (this path is rare).
      float sfx[TPL][4], run[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) run[j] = 1.f;
#pragma unroll
      for (int u = TPL - 1; u >= 0; --u) {
        const int tok = tb0 + u;
        float al[4];
        gate4(min(tok, L - 1), c0, al, false);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sfx[u][j] = run[j];
          run[j] *= tok < L ? al[j] : 1.f;
        }
      }
      float later[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) later[j] = 1.f;
      for (int d = 1; d < TH; ++d) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float y = __shfl(run[j], l + d * CG);
          if (th + d < TH) later[j] *= y;
        }
      }
#pragma unroll
      for (int u = 0; u < TPL; ++u) {
        float kt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) kt[j] = kval(u, j) * sfx[u][j] * later[j] * gb[j];
        ktt[u] = F4::pack(kt);
      }
    }
    __syncthreads();

    // ---- fast path: R^T and A^T tiles on the matrix cores.  Pair (I, J),
    // I >= J: D[j][i] over j in block J (rows), i in block I (columns).
    constexpr int NP = 3;  // pairs per wave: w, w + 4, w + 8 (< 10)
    f32x4 rt[NP], at[NP];
    if (!exact) {
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        const int p = w + 4 * s;
        rt[s] = at[s] = zero4();
        if (p < 10) {
          int I, J;
          tile_ij(p, I, J);
#pragma unroll
          for (int u = 0; u < LK::F::NU; ++u) {
            const char *ad = sKd + LK::slot_off(J, u, l & 15, l >> 4);
            rt[s] = slot_mma<E, DK>(ad, sKh + LK::slot_off(I, u, l & 15, l >> 4), rt[s]);
            at[s] = slot_mma<E, DK>(ad, sQh + LK::slot_off(I, u, l & 15, l >> 4), at[s]);
          }
        }
      }
    }
    copy_out<LK>(rec + a.lay.kh, sKh);
    copy_out<LK>(rec + a.lay.qh, sQh);
    __syncthreads();  // phase-1 images are dead from here on

    E *gA = reinterpret_cast<E *>(rec + a.lay.aqk);
    if (!exact) {
      // R (scaled by beta_i, j < i) to LDS for the solve; A (j <= i) straight to
      // the record: lane (i, g) holds A[i][16J + 4g .. +3], four consecutive
      // elements of one record slot.
#pragma unroll
      for (int s = 0; s < NP; ++s) {
        const int p = w + 4 * s;
        if (p < 10) {
          int I, J;
          tile_ij(p, I, J);
          const int i = 16 * I + (l & 15), jb = 16 * J + 4 * (l >> 4);
          float rv[4], av[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            rv[r] = jb + r < i ? sBeta[i] * rt[s][r] : 0.f;
            av[r] = jb + r < i ? at[s][r] : (jb + r == i ? (diag_exact ? sDiag[i] : at[s][r]) : 0.f);
          }
          *reinterpret_cast<f32x4 *>(sR + i * LDR + jb) = f32x4{rv[0], rv[1], rv[2], rv[3]};
          *reinterpret_cast<typename F4::vec *>(gA + tri_index<E>(i, jb)) = F4::pack(av);
        }
      }
      // blocks above the diagonal of A that share a stored slab with the
      // diagonal are zero
      for (int idx = tid; idx < 16 * 64; idx += kThreads) {
        const int I = idx >> 8, J = (idx >> 6) & 3, ln = idx & 63;
        if (J > I && 16 * J / FragShape<E, 64>::W < tri_slabs(I, (int)sizeof(E))) {
          const float z[4] = {0.f, 0.f, 0.f, 0.f};
          *reinterpret_cast<typename F4::vec *>(gA + tri_index<E>(16 * I + (ln & 15), 16 * J + 4 * (ln >> 4))) =
              F4::pack(z);
        }
      }
      // Kend^T into its LDS image (copied out after the next barrier): four
      // consecutive tokens of one channel are contiguous there
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (TPL >= 4) {
#pragma unroll
          for (int u = 0; u < TPL; u += 4) {
            typename F4::vec v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const E x = ktt[u + e][j];
              v[e] = x;
            }
            *reinterpret_cast<typename F4::vec *>(sX + LT::elem_off(c0 + j, tb0 + u)) = v;
          }
        } else {
#pragma unroll
          for (int u = 0; u < TPL; ++u) {
            const E x = ktt[u][j];
            *reinterpret_cast<E *>(sX + LT::elem_off(c0 + j, tb0 + u)) = x;
          }
        }
      }
    } else {
      // R and A channel by channel: thread (j, part) runs D_{j+1:i} over i for
      // CQ channels; the NQ parts of row j sit in neighbouring lanes and are
      // summed across them.  At most 16 channels per lane keep the running
      // products in few registers (this path is rare: with more channels per
      // lane its registers would push values of the common path into
      // scratch); with NQ > 4 the 64 rows take NQ/4 passes.
      constexpr int CQ = DK / 4 > 16 ? 16 : DK / 4;
      constexpr int NQ = DK / CQ;          // lanes per row
      constexpr int JP = kThreads / NQ;    // rows per pass
      float *sA = reinterpret_cast<float *>(sX);
      const int qd = tid % NQ;
#pragma unroll 1
      for (int jb = 0; jb < kChunk; jb += JP) {
        const int j = jb + tid / NQ;
        const size_t cb = (size_t)t0 * hs + (size_t)h * DK + qd * CQ;
        float kj[CQ], rho[CQ];
#pragma unroll
        for (int cc = 0; cc < CQ; cc += 4) {
          if constexpr (CONV)
            conv_load4(k, a.conv_k, min(j, L - 1), qd * CQ + cc, kj + cc);
          else
            F4::load(k + cb + (size_t)min(j, L - 1) * hs + cc, kj + cc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (ACTQK) kj[cc + e] = (float)(E)(silu_f(kj[cc + e]) * sInvNorm[0][min(j, L - 1)]);
            kj[cc + e] = j < L ? kj[cc + e] : 0.f;
            rho[cc + e] = 1.f;
          }
        }
        for (int i = 0; i < kChunk; ++i) {
          const bool live = i < L;
          const size_t off = cb + (size_t)min(i, L - 1) * hs;
          float racc = 0.f, aacc = 0.f;
#pragma unroll
          for (int cc = 0; cc < CQ; cc += 4) {
            float al[4], kx[4], qx[4];
            gate4(min(i, L - 1), qd * CQ + cc, al, false);
            if constexpr (CONV) {
              // the taps are read again for every token: kept live across the
              // loop, those of all channel groups would not fit in registers
              __asm__ volatile("" ::: "memory");
              conv_load4(k, a.conv_k, min(i, L - 1), qd * CQ + cc, kx);
              conv_load4(q, a.conv_q, min(i, L - 1), qd * CQ + cc, qx);
            } else {
              F4::load(k + off + cc, kx);
              F4::load(q + off + cc, qx);
            }
            if constexpr (ACTQK) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                // rounded to E like the activated values of the fast path
                kx[e] = (float)(E)(silu_f(kx[e]) * sInvNorm[0][min(i, L - 1)]);
                qx[e] = (float)(E)(silu_f(qx[e]) * sInvNorm[1][min(i, L - 1)]);
              }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (i > j) rho[cc + e] *= live ? al[e] : 1.f;
              const float wgt = i >= j ? kj[cc + e] * rho[cc + e] : 0.f;
              racc += (live ? kx[e] : 0.f) * wgt;
              aacc += (live ? qx[e] : 0.f) * wgt;
            }
          }
          racc = group_sum<NQ>(racc);
          aacc = group_sum<NQ>(aacc);
          if (qd == 0) {
            sR[i * LDR + j] = i > j ? sBeta[i] * racc : 0.f;
            sA[i * LDR + j] = i >= j ? a.scale * aacc : 0.f;
          }
        }
      }
      // Kend^T straight to the record (scattered; this path is rare)
      E *gT = reinterpret_cast<E *>(rec + a.lay.ktt);
#pragma unroll
      for (int u = 0; u < TPL; ++u)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const E x = ktt[u][jj];
          gT[frag_index<E, 64>(c0 + jj, tb0 + u)] = x;
        }
    }
    __syncthreads();

    if (w == 0 && th == 0) *reinterpret_cast<f32x4 *>(rec + a.lay.p63 + 4 * c0) = f32x4{p63[0], p63[1], p63[2], p63[3]};

    // ---- T = (I + R)^{-1}.  Wave 0 inverts the four diagonal 16x16 blocks by
    // forward substitution while waves 1-3 copy Kend^T (or A) out; then three
    // levels of off-diagonal blocks, T_IJ = -T_II sum_K R_IK T_KJ, and the
    // waves a level leaves idle write the row tiles of Tb = T Diag(beta) whose
    // blocks are final.
    E *gTb = reinterpret_cast<E *>(rec + a.lay.tb);
    if (w == 0) {
      const int b = l >> 4, jc = l & 15;
      float X[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        float s = m == jc ? 1.f : 0.f;
#pragma unroll
        for (int p = 0; p < m; ++p) s -= sR[(16 * b + m) * LDR + 16 * b + p] * X[p];
        X[m] = s;
      }
#pragma unroll
      for (int m = 0; m < 16; ++m) sT[(16 * b + m) * LDR + 16 * b + jc] = X[m];
    } else if (!exact) {
      copy_out<LT>(rec + a.lay.ktt, sX, 64, kThreads - 64);
    } else {
      tile64_out<E, LDR>(gA, reinterpret_cast<const float *>(sX), nullptr, 0, 4, 64, kThreads - 64);
    }
    __syncthreads();
    if (w < 3) inverse_offdiag_block<LDR>(w + 1, w, sR, sT);  // (1,0) (2,1) (3,2)
    else tile64_out<E, LDR>(gTb, sT, sBeta, 0, 1, 192, 64);     // row tile 0 is final
    __syncthreads();
    if (w < 2) inverse_offdiag_block<LDR>(w + 2, w, sR, sT);  // (2,0) (3,1)
    else tile64_out<E, LDR>(gTb, sT, sBeta, 1, 2, 128, 128);    // row tile 1
    __syncthreads();
    if (w == 0) inverse_offdiag_block<LDR>(3, 0, sR, sT);     // (3,0)
    else tile64_out<E, LDR>(gTb, sT, sBeta, 2, 3, 64, 192);     // row tile 2
    __syncthreads();
    tile64_out<E, LDR>(gTb, sT, sBeta, 3, 4);                   // row tile 3

    // CONV: v's convolution into this chunk's rows of o; a thread takes a run
    // of four tokens and 16 bytes of channels (its window: the seven rows
    // ending at the run's last token)
    if constexpr (CONV) {
      typedef typename Row16<E>::vec RV;
      constexpr int VE = Row16<E>::N, NW = 4 + kConvTaps - 1;
      const int GR = a.dv / VE;  // 16-byte groups per row
      const E *V = reinterpret_cast<const E *>(a.v);
      E *O = reinterpret_cast<E *>(a.o);
      const size_t vs = (size_t)a.H * a.dv;
      for (int idx = tid; idx < (kChunk / 4) * GR; idx += kThreads) {
        const int r0 = 4 * (idx / GR), ch = (idx % GR) * VE;
        if (r0 >= L) continue;
        RV win[NW];
        unsigned okm = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
          const int rel = min(r0 - (kConvTaps - 1) + i, L - 1);
          const bool ok = t0 + rel >= s0;
          okm |= (unsigned)ok << i;
          win[i] = __builtin_nontemporal_load(
              reinterpret_cast<const RV *>(V + (size_t)(t0 + (ok ? rel : 0)) * vs + (size_t)h * a.dv + ch));
        }
        f32x4 wt[VE];
#pragma unroll
        for (int j = 0; j < VE; ++j)
          wt[j] = *reinterpret_cast<const f32x4 *>(a.conv_v + ((size_t)h * a.dv + ch + j) * kConvTaps);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (r0 + u >= L) break;
          RV y;
#pragma unroll
          for (int j = 0; j < VE; ++j) {
            float xv[kConvTaps];
#pragma unroll
            for (int i = 0; i < kConvTaps; ++i) xv[i] = (okm >> (u + i)) & 1 ? (float)win[u + i][j] : 0.f;
            y[j] = (E)conv_taps(wt[j], xv[0], xv[1], xv[2], xv[3]);
          }
          __builtin_nontemporal_store(y, reinterpret_cast<RV *>(O + (size_t)(t0 + r0 + u) * vs + (size_t)h * a.dv + ch));
        }
      }
    }
  };

  if constexpr (!SCHED) {
    // heads fastest: the workgroups of one chunk run together, so the lines
    // they share (each token's beta row holds every head's) are fetched once,
    // and they read neighbouring parts of the same token rows (measured
    // against chunks fastest: packed workload 3249 -> 2999 us per call,
    // long-context two-phase 2260 -> 2147, 32 x 256 chunks 593 -> 551; the
    // prefill workload 104 -> 103)
    prep_one(blockIdx.x / a.H, blockIdx.x % a.H);
    return;
  }
  // Overlapped schedule (a separate instantiation): records of the units
  // u = x (mod 8) are prepared on XCD x, chunk-major (chunk 0 of every such
  // unit first).  A workgroup takes the next task from its XCD's counter (the
  // dispatcher deals workgroups to the eight XCDs in turn, and the grid holds
  // eight times the largest per-XCD task count, so every task is taken), and
  // publishes the finished record by setting bit ci % 32 of the unit's ready
  // word ci / 32 once its stores have reached L2.
  __shared__ int sTask;
  const int x = xcd_id();
  const int nux = a.n_units > x ? (a.n_units - x + 7) / 8 : 0;
  if (threadIdx.x == 0)
    sTask = __hip_atomic_fetch_add(a.ctl + kCtlPrepNext + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const int t = sTask;
  if (t >= nux * a.src.nct) return;
  const int u = x + 8 * (t % nux), ci = t / nux;
  const long long slot = (long long)(u / a.H) * a.src.nct + ci;
  prep_one(slot, u % a.H);
  // the producing XCD, in the record's padding after D_{0:63}; the scan
  // checks it against its own (the record is read through this XCD's L2)
  if (threadIdx.x == 0)
    *reinterpret_cast<int *>(a.ws_records + ((size_t)slot * a.H + u % a.H) * a.lay.bytes + a.lay.p63 + DK * 4) = x;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's record stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_or(a.ready + (size_t)u * a.ready_words + (ci >> 5), 1 << (ci & 31), __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_AGENT);
}

template <int DK, typename E, int GATE, bool ACTQK, bool SCHED = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void chunk_prep_kernel(PrepKArgs a) {
  chunk_prep_body<DK, E, GATE, ACTQK, SCHED, false>(a);
}

// With the convolution the prep holds each lane's window of raw rows and the
// taps besides its usual values: at three waves per SIMD that spilled up to
// 39 registers; at two it spills none and was faster (prefill workload with
// the block's operations: 102.4 -> 95.6 us per prep; the prep without the
// convolution went the other way, 63.0 -> 70.5, so it keeps three).
template <int DK, typename E, int GATE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void chunk_prep_conv_kernel(PrepKArgs a) {
  chunk_prep_body<DK, E, GATE, true, false, true>(a);
}

// ======================================================= kernel 2: chunk scan
struct ScanKArgs {
  const void *v;
  const float *S0;
  void *o;
  float *S_final;
  const char *ws_records;
  ChunkRecordLayout lay;
  int H, dv, T, nct;
  const int32_t *seq_tok0, *seq_chunk0;  // packed batch tables, or null
  const int32_t *seq_order;              // packed: sequences longest first (unit u -> sequence seq_order[u / H])
  float scale;
  int n_units;                           // sequences * heads
  int wg_per_unit;                       // workgroups per unit (value tiles / waves per WG)
  // control words (both schedules: the two-phase scan records its schedule
  // there); overlapped schedule only: ready words (ready_words per unit, bit
  // c % 32 of word c / 32 set once chunk c's record is in L2)
  const int *ready;
  int ready_words;
  int *ctl;
  long long wait_ticks;  // bound on one ready-flag wait (100 MHz ticks; 0: give up at once)
  // two-phase only: pull each chunk record into L2 a step before it is
  // copied to LDS (set when the records outgrow the 256 MB Infinity Cache,
  // so they come from HBM)
  int touch_ahead;
  // split-sequence scan (two-phase kernels): the packed sequences are
  // segments, seg_per_seq of them per sequence; the last segment's end state
  // goes to S_last (the sequence's final state) and the others' are not
  // stored; sched_id is the schedule word the call records (0: two-phase)
  float *S_last;
  int seg_per_seq;
  int sched_id;
};

// B operands built from accumulator tiles.  Tile q of a K x 16 operand holds
// rows 16q..16q+15; lane l has rows 4g..4g+3 (g = l/16) of column l%16, which
// is exactly the k order of the fragment-ordered A operands (FragShape).
template <typename E, int K> struct BOps;

template <int K> struct BOps<bf16, K> {
  typedef FragShape<bf16, K> F;
  typedef typename std::conditional<F::wide, bf16x8, bf16x4>::type frag;
  frag f[F::NU];
  __device__ __forceinline__ void build(const f32x4 *t) {
#pragma unroll
    for (int u = 0; u < F::NU; ++u) {
      if constexpr (F::wide) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f[u][r] = (bf16)t[2 * u][r];
          f[u][4 + r] = (bf16)t[2 * u + 1][r];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) f[u][r] = (bf16)t[u][r];
      }
    }
  }
  // A fragments of one 16-row tile (k < KU, whole slabs); `a` points at the
  // tile's first fragment.
  template <int KU> struct A {
    frag x[(KU + F::W - 1) / F::W];
  };
  template <int KU>
  __device__ __forceinline__ static A<KU> load(const bf16 *a) {
    A<KU> r;
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < (KU + F::W - 1) / F::W; ++u) r.x[u] = *reinterpret_cast<const frag *>(a + (u * 64 + l) * F::KS);
    return r;
  }
  // acc += A(16 rows, k < KU) * B(k < KU); columns beyond KU are zero
  template <int KU>
  __device__ __forceinline__ f32x4 mma(const A<KU> &a, f32x4 acc) const {
#pragma unroll
    for (int u = 0; u < (KU + F::W - 1) / F::W; ++u) acc = mma1(a.x[u], u, acc);
    return acc;
  }
  // one slab: the A fragment of slab u of the tile at `a`, and its product
  __device__ __forceinline__ static frag load1(const bf16 *a, int u) {
    return *reinterpret_cast<const frag *>(a + (u * 64 + lane_id()) * F::KS);
  }
  __device__ __forceinline__ f32x4 mma1(const frag &a, int u, f32x4 acc) const {
    if constexpr (F::wide)
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, f[u], acc, 0, 0, 0);
    else
      return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, f[u], acc, 0, 0, 0);
  }
};

template <int K> struct BOps<float, K> {
  typedef FragShape<float, K> F;
  f32x4 f[F::NU];
  __device__ __forceinline__ void build(const f32x4 *t) {
#pragma unroll
    for (int u = 0; u < F::NU; ++u) f[u] = t[u];
  }
  template <int KU> struct A {
    f32x4 x[(KU + 15) / 16];
  };
  template <int KU>
  __device__ __forceinline__ static A<KU> load(const float *a) {
    A<KU> r;
    const int l = lane_id();
#pragma unroll
    for (int u = 0; u < (KU + 15) / 16; ++u) r.x[u] = *reinterpret_cast<const f32x4 *>(a + (u * 64 + l) * 4);
    return r;
  }
  template <int KU>
  __device__ __forceinline__ f32x4 mma(const A<KU> &a, f32x4 acc) const {
#pragma unroll
    for (int u = 0; u < (KU + 15) / 16; ++u) acc = mma1(a.x[u], u, acc);
    return acc;
  }
  typedef f32x4 frag;
  __device__ __forceinline__ static frag load1(const float *a, int u) {
    return *reinterpret_cast<const f32x4 *>(a + (u * 64 + lane_id()) * 4);
  }
  __device__ __forceinline__ f32x4 mma1(const frag &a, int u, f32x4 acc) const {
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], f[u][s], acc, 0, 0, 0);
    return acc;
  }
};

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + 16 l (global_load_lds_dwordx4; the LDS base goes through M0).
// M0 is written here and nowhere else in the kernels that call this.
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);  // wave-uniform by construction
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}

// 4 bytes per lane from global memory into LDS (global_load_lds_dword; lane
// l's bytes land at lds_base + 4 l).  Used only to pull lines into L2 ahead
// of their copy: the LDS bytes are a landing place nothing reads.
__device__ __forceinline__ void lds_dma4(const void *src, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}

// Pulls 8 KiB blocks b0, b0 + 1, .., b0 + NB - 1 of a record (of `bytes`
// bytes) into L2: one line of 128 bytes per lane, addresses clamped to the
// record; the data lands in a 256-byte LDS scratch that nobody reads.
template <int NB>
__device__ __forceinline__ void touch_record(const char *rec, int bytes, int b0, uint32_t scratch_lds) {
#pragma unroll
  for (int i = 0; i < NB; ++i) lds_dma4(rec + min((b0 + i) * 8192 + lane_id() * 128, bytes - 4), scratch_lds);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt[3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).  Vector memory loads
// retire in issue order, so this waits for all but the N latest.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same with the nontemporal hint, for data read exactly once.
__device__ __forceinline__ void lds_dma16_nt(const void *src, uint32_t lds_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(lds_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
               :
               : "v"(src), "s"(base)
               : "memory", "m0");
}

// Compile-time copy of ChunkRecordLayout for the scan's LDS image of a record.
template <int DK, typename E> struct RecordShape {
  static constexpr int es = sizeof(E);
  static constexpr int kh = 0, qh = 64 * DK * es, ktt = 128 * DK * es, tb = 192 * DK * es;
  static constexpr int aqk = tb + (int)tri_bytes(es), p63 = aqk + (int)tri_bytes(es);
  static constexpr int bytes = (p63 + DK * 4 + 1023) / 1024 * 1024;
};

// One chunk of the scan for one compute wave, which owns 16*NT value columns
// and keeps S^T (d_k x 16*NT) in fp32 accumulator tiles st[d_k/16][NT]:
//   X_top = Kbnd S^T, X_bot = s Qbnd S^T, Ebar = V - X_top, E = Tb Ebar,
//   O = X_bot + A E (into ov), S^T <- D_{0:63} S^T + Kend^T E.
// `recb` is the chunk's record image in LDS; `vs` points at the wave's first
// value column of the chunk's value tile in LDS (row stride VSTRIDE
// elements).  Every product loop runs slab-major (the k slab outer, the
// 16-row tiles inner), so consecutive matrix-core products are independent
// and none waits for the previous one's result; the LDS operand reads of
// later phases are issued early, in the order they are used.
// OUT = false: the state update alone (no X_bot, no outputs; s Qbnd and A
// are not read).  VZERO: V = 0 (vs is not read).
template <int DK, typename E, int NT, int VSTRIDE, bool OUT = true, bool VZERO = false>
__device__ __forceinline__ void scan_chunk(const char *recb, const E *vs, f32x4 (*st)[NT], f32x4 (*ov)[NT]) {
  typedef RecordShape<DK, E> RS;
  typedef FragShape<E, DK> FK;   // products over d_k
  typedef FragShape<E, 64> FT;   // products over the 64 tokens
  constexpr int CT = DK / 16;
  constexpr int TILE_K = FK::NU * 64 * FK::KS;   // elements per 16-row tile, K = d_k
  constexpr int TILE_T = FT::NU * 64 * FT::KS;   // elements per 16-row tile, K = 64
  const int l = lane_id(), col = l & 15, g = l >> 4;
  typedef BOps<E, DK> BK;
  typedef BOps<E, 64> BT;
  constexpr int UK = FK::NU, UT = FT::NU;          // slabs over d_k, over 64 tokens
  const E *Kh = reinterpret_cast<const E *>(recb + RS::kh);
  const E *Qh = reinterpret_cast<const E *>(recb + RS::qh);
  const E *KtT = reinterpret_cast<const E *>(recb + RS::ktt);
  const E *Tb = reinterpret_cast<const E *>(recb + RS::tb);
  const E *Aq = reinterpret_cast<const E *>(recb + RS::aqk);
  const float *P63 = reinterpret_cast<const float *>(recb + RS::p63);
  // row tile I of Tb and A only needs slabs holding columns < 16 (I + 1)
  auto need = [](int I, int u) { return u * FT::W < 16 * (I + 1); };

  // B operands from the state; X_top = Kbnd S^T, X_bot = s Qbnd S^T
  BK sb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 col_tiles[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) col_tiles[ct] = st[ct][nt];
    sb[nt].build(col_tiles);
  }
  f32x4 xt[4][NT], xb[4][NT];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) xt[I][nt] = xb[I][nt] = zero4();
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    typename BK::frag fk[4], fq[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      fk[I] = BK::load1(Kh + I * TILE_K, u);
      if constexpr (OUT) fq[I] = BK::load1(Qh + I * TILE_K, u);
    }
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        xt[I][nt] = sb[nt].mma1(fk[I], u, xt[I][nt]);
        if constexpr (OUT) xb[I][nt] = sb[nt].mma1(fq[I], u, xb[I][nt]);
      }
  }
  // operands of the later phases
  typename BT::frag ftb[4][UT], faq[4][UT], fkt[CT][UT];
  float vv[NT][4][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vv[nt][I][r] = VZERO ? 0.f : to_f(vs[(16 * I + 4 * g + r) * VSTRIDE + 16 * nt + col]);
#pragma unroll
  for (int u = 0; u < UT; ++u)
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if (need(I, u)) ftb[I][u] = BT::load1(Tb + tri_slab0(I, (int)sizeof(E)) * 64 * FT::KS, u);
  if constexpr (OUT) {
#pragma unroll
    for (int u = 0; u < UT; ++u)
#pragma unroll
      for (int I = 0; I < 4; ++I)
        if (need(I, u)) faq[I][u] = BT::load1(Aq + tri_slab0(I, (int)sizeof(E)) * 64 * FT::KS, u);
  }
#pragma unroll
  for (int u = 0; u < UT; ++u)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) fkt[ct][u] = BT::load1(KtT + ct * TILE_T, u);
  f32x4 p[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) p[ct] = *reinterpret_cast<const f32x4 *>(P63 + 16 * ct + 4 * g);

  // Ebar = V - X_top ; E = Tb Ebar
  BT ebo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 eb[4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) eb[I][r] = vv[nt][I][r] - xt[I][nt][r];
    ebo[nt].build(eb);
  }
  f32x4 e[4][NT];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) e[I][nt] = zero4();
#pragma unroll
  for (int u = 0; u < UT; ++u)
#pragma unroll
    for (int I = 0; I < 4; ++I)
      if (need(I, u))
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) e[I][nt] = ebo[nt].mma1(ftb[I][u], u, e[I][nt]);
  // O = s Qbnd S^T + A E ;  S^T = D_{0:63} S^T + Kend^T E
  BT eo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 et[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) et[I] = e[I][nt];
    eo[nt].build(et);
  }
  if constexpr (OUT) {
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) ov[I][nt] = xb[I][nt];
  }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[ct][nt][r] *= p[ct][r];
#pragma unroll
  for (int u = 0; u < UT; ++u) {
    if constexpr (OUT) {
#pragma unroll
      for (int I = 0; I < 4; ++I)
        if (need(I, u))
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) ov[I][nt] = eo[nt].mma1(faq[I][u], u, ov[I][nt]);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st[ct][nt] = eo[nt].mma1(fkt[ct][u], u, st[ct][nt]);
  }
}

// Scan.  A workgroup serves one unit (sequence, head): CW compute waves, each
// owning 16*NT value columns and keeping S^T (d_k x 16*NT) in fp32
// accumulator tiles, plus one copy wave that streams the chunk records (and
// the compute waves' value slices) into a double-buffered LDS image with
// global_load_lds, so the compute waves never issue memory loads.  While the
// compute waves work on chunk c, the copy wave fills the other buffer with
// chunk c+1; one workgroup barrier per chunk hands the buffers over.  Each
// product takes its A operand from the LDS record (fragment order:
// conflict-free 16-byte reads, shared by the NT column tiles) and its B
// operand from the wave's own accumulators.  Workgroups of one unit get ids
// congruent mod 8, which the dispatcher sends to one XCD.
template <int DK, typename E, int NT, int CW, int NCP, bool SCHED = false>
__global__ __launch_bounds__(64 * (CW + NCP)) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunk_scan_kernel(ScanKArgs a) {
  typedef RecordShape<DK, E> RS;
  constexpr int CT = DK / 16;
  constexpr int VC = 16 * NT;                   // value columns per compute wave
  typedef FragShape<E, DK> FK;   // products over d_k
  typedef FragShape<E, 64> FT;   // products over the 64 tokens
  constexpr int TILE_K = FK::NU * 64 * FK::KS;   // elements per 16-row tile, K = d_k
  constexpr int TILE_T = FT::NU * 64 * FT::KS;   // elements per 16-row tile, K = 64
  constexpr int VSL = 64 * VC;                   // value-slice elements per compute wave
  constexpr int VBYTES = CW * VSL * (int)sizeof(E);
  // outputs of a chunk, staged as rows for the copy waves to store: WC
  // columns per row, rows padded by 16 bytes
  constexpr int OROW = CW * VC * (int)sizeof(E) + 16;
  // records double-buffered, value tiles in a ring of three (they come from
  // HBM, so they are requested two chunks ahead) and two output stages, if
  // that fits
  constexpr int NBUF = 2 * RS::bytes + 3 * VBYTES + 2 * 64 * OROW <= 159 * 1024 ? 2 : 1;
  static_assert(RS::bytes + VBYTES <= 159 * 1024, "one stage must fit in LDS");
  constexpr int NV = NBUF == 2 ? 3 : 1;
  __shared__ __attribute__((aligned(1024))) char rec0[RS::bytes];
  __shared__ __attribute__((aligned(1024))) char rec1[NBUF == 2 ? RS::bytes : 1024];
  __shared__ __attribute__((aligned(16))) E vring[NV][CW * VSL];
  __shared__ __attribute__((aligned(16))) char otile[2][NBUF == 2 ? 64 * OROW : 16];
  __shared__ __attribute__((aligned(16))) char touch_area[256];

  const int w = wave_id(), l = lane_id(), col = l & 15, g = l >> 4;
  int u, grp;  // unit and value-column group of this workgroup
  const int x = SCHED ? xcd_id() : 0;
  if constexpr (SCHED) {
    // overlapped schedule: the next (unit, group) ticket of this XCD, whose
    // prep workers produce the records of units u = x (mod 8)
    __shared__ int sTicket;
    if (threadIdx.x == 0)
      sTicket = __hip_atomic_fetch_add(a.ctl + kCtlScanNext + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    u = x + 8 * (sTicket / a.wg_per_unit);
    grp = sTicket % a.wg_per_unit;
  } else {
    const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
    u = (slot / a.wg_per_unit) * 8 + xcd;
    grp = slot % a.wg_per_unit;
    // the schedule this call ran, and no schedule errors
    if (bid == 0 && threadIdx.x == 0) {
      a.ctl[kCtlSchedule] = a.sched_id ? a.sched_id : kScheduleTwoPhase;
      a.ctl[kCtlError] = 0;
    }
  }
  if (u >= a.n_units) return;
  const int n = a.seq_order ? a.seq_order[u / a.H] : u / a.H, h = u % a.H;
  const int vwg = grp * (CW * VC);  // first value column of the workgroup
  const int H = a.H, DV = a.dv;
  const bool copier = w >= CW;
  const int cpi = w - CW;                  // index among the copy waves
  const bool vcopier = w == CW + NCP - 1;  // the copy wave that also moves the value tiles

  long long tstart, ntok, chunk0;
  if (a.seq_tok0) {
    tstart = a.seq_tok0[n];
    ntok = a.seq_tok0[n + 1] - tstart;
    chunk0 = a.seq_chunk0[n];
  } else {
    tstart = (long long)n * a.T;
    ntok = a.T;
    chunk0 = (long long)n * a.nct;
  }
  const int nchunks = (int)((ntok + kChunk - 1) / kChunk);
  const E *V = reinterpret_cast<const E *>(a.v);
  E *O = reinterpret_cast<E *>(a.o);
  const size_t tok_stride = (size_t)H * DV;

  // ----------------------------------------------------------- copy wave
  // The workgroup's value columns land as [token][WC elements] (RB bytes per
  // row).  Each copy covers 64/LPRW whole rows, LPRW lanes per row, so one
  // instruction touches one line segment per row instead of one line per
  // lane.  Rows past the end of the sequence repeat its last token (they never
  // reach a valid output: their Tb rows and columns are zero).
  constexpr int VE = 16 / (int)sizeof(E);        // elements per 16-byte group
  constexpr int WC = CW * VC;                    // value columns of the workgroup
  constexpr int RB = WC * (int)sizeof(E);        // bytes per staged row
  constexpr int LPRW = RB / 16;                  // lanes per row
  constexpr int RPI = 64 / LPRW;                 // rows per copy
  static_assert(RB % 16 == 0 && LPRW <= 64, "value rows are whole 16-byte groups");
  constexpr int NVD = 64 / RPI;                  // value copies per chunk
  auto copy_rec = [&](int ci, char *rec) {
    const char *src = a.ws_records + ((size_t)(chunk0 + ci) * H + h) * RS::bytes + l * 16;
    const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)rec;
    // copy wave cpi takes KiB blocks cpi*QPW .. cpi*QPW + QPW - 1, clamped to
    // the last block (a clamped block is copied twice with the same bytes),
    // so the loop unrolls with no branch per copy
    constexpr int NQ = RS::bytes / 1024, QPW = (NQ + NCP - 1) / NCP;
#pragma unroll
    for (int qq = 0; qq < QPW; ++qq) {
      const int q = min(cpi * QPW + qq, NQ - 1);
      lds_dma16(src + q * 1024, lds + q * 1024);
    }
  };
  auto copy_v = [&](int ci, E *vsl) {
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const uint32_t vl = (uint32_t)(size_t)(__attribute__((address_space(3))) E *)vsl;
    const int vr = l / LPRW, vc = (l % LPRW) * VE;
#pragma unroll
    for (int j = 0; j < 64 / RPI; ++j) {
      const E *vsrc = V + (size_t)(t0 + min(j * RPI + vr, L - 1)) * tok_stride + (size_t)h * DV + vwg + vc;
      lds_dma16_nt(vsrc, vl + j * 1024);
    }
  };
  // chunk ci's outputs from an LDS stage to o: 16-byte row segments; the
  // buffer descriptor covers exactly the chunk's valid rows, so rows past the
  // end of the sequence are dropped by the hardware (the whole offset goes in
  // the VGPR operand: the range check of a raw buffer access does not include
  // soffset); nontemporal, every output byte is written once
  auto store_tile = [&](int ci, const char *ot) {
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        O + (size_t)t0 * tok_stride, 0, (int)((size_t)L * tok_stride * sizeof(E)), 0x00020000);
    constexpr int SEG = RB / 16;
#pragma unroll
    for (int k = 0; k < SEG; ++k) {
      const int idx = l + 64 * k, row = idx / SEG, sg = idx % SEG;
      const f32x4 v = *reinterpret_cast<const f32x4 *>(ot + row * OROW + sg * 16);
      const int off = (int)(((size_t)row * tok_stride + (size_t)h * DV + vwg) * sizeof(E)) + sg * 16;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((__vector_size__(16))) unsigned int, v),
                                             rs, off, 0, 2);
    }
  };
  // Overlapped schedule: chunk ci's record may be copied once bit ci % 32 of
  // the unit's ready word ci / 32 is set.  Lane 0 reads the word (bypassing
  // the CU's L1: agent-scope load) only when the bit is not known yet; a wait
  // longer than a.wait_ticks (1.3 s by default: the prep could not run) sets
  // kSchedErrTimeout and the wave stops waiting: the results are then wrong,
  // but the kernel always finishes.  A bound of 0 gives up without reading.
  unsigned known = 0;
  int known_word = -1;
  bool gave_up = false;
  auto wait_rec = [&](int ci) {
    if constexpr (SCHED) {
      const int wd = ci >> 5;
      const unsigned bit = 1u << (ci & 31);
      if (wd != known_word) {
        known_word = wd;
        known = 0;
      }
      if ((known & bit) || gave_up) return;
      if (a.wait_ticks <= 0) {
        if (l == 0) __hip_atomic_fetch_or(a.ctl + kCtlError, kSchedErrTimeout, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        gave_up = true;
        return;
      }
      const int *word = a.ready + (size_t)u * a.ready_words + wd;
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        unsigned v = 0;
        if (l == 0) v = (unsigned)__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        known = __builtin_amdgcn_readfirstlane(v);
        if (known & bit) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > (unsigned long long)a.wait_ticks) {  // 100 MHz ticks
          if (l == 0) __hip_atomic_fetch_or(a.ctl + kCtlError, kSchedErrTimeout, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
          gave_up = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
  };
  if (copier) {
    if (NBUF == 2) {
      if (nchunks > 0) {
        wait_rec(0);
        copy_rec(0, rec0);
        if (vcopier) copy_v(0, vring[0]);
      }
      if (vcopier && nchunks > 1) {
        copy_v(1, vring[1]);
        wait_vmcnt<NVD>();             // chunk 0 in; chunk 1's values may still fly
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();  // chunk 0 ready
      for (int ci = 0; ci < nchunks; ++ci) {
        // record buffer (ci+1)%2 and value slot (ci+2)%3 held chunk ci-1, which
        // every compute wave finished before the barrier that ended the
        // previous step
        if (ci + 1 < nchunks) {
          wait_rec(ci + 1);
          copy_rec(ci + 1, (ci & 1) ? rec0 : rec1);
        }
        // the compute waves staged chunk ci-1's outputs before the last barrier
        if (cpi == 0 && ci > 0) store_tile(ci - 1, otile[(ci - 1) & 1]);
        if (!SCHED && a.touch_ahead && cpi == 1 && !vcopier && ci + 2 < nchunks) {
          // record ci+2 into L2: this workgroup's share, two 8 KiB blocks
          touch_record<2>(a.ws_records + ((size_t)(chunk0 + ci + 2) * H + h) * RS::bytes, RS::bytes, 2 * grp,
                          (uint32_t)(size_t)(__attribute__((address_space(3))) char *)touch_area);
          wait_vmcnt<2>();             // the copies; the touches may still fly
        } else if (vcopier && ci + 2 < nchunks) {
          copy_v(ci + 2, vring[(ci + 2) % 3]);
          wait_vmcnt<NVD>();           // all but chunk ci+2's values
        } else {
          __builtin_amdgcn_s_waitcnt(0);
        }
        __syncthreads();  // chunk ci done by the compute waves, chunk ci+1 ready
      }
      if (cpi == 0 && nchunks > 0) store_tile(nchunks - 1, otile[(nchunks - 1) & 1]);
    } else {
      for (int ci = 0; ci < nchunks; ++ci) {
        __syncthreads();  // buffer free
        copy_rec(ci, rec0);
        if (vcopier) copy_v(ci, vring[0]);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // buffer ready
      }
    }
    return;
  }

  // -------------------------------------------------------- compute waves
  const int v0 = vwg + w * VC;
  const size_t sbase = ((size_t)n * H + h) * DV * DK + (size_t)(v0 + col) * DK;
  f32x4 st[CT][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      st[ct][nt] = a.S0 ? *reinterpret_cast<const f32x4 *>(a.S0 + sbase + (size_t)16 * nt * DK + 16 * ct + 4 * g)
                        : zero4();

  auto compute = [&](const char *recb, const E *vs, f32x4 (*ov)[NT]) {
    if constexpr (SCHED) {
      // the record must come from this XCD's prep workers (stamped by them)
      static_assert(RS::p63 + DK * 4 + 4 <= RS::bytes, "room for the XCD stamp");
      if (w == 0 && l == 0 && *reinterpret_cast<const int *>(recb + RS::p63 + DK * 4) != x)
        __hip_atomic_fetch_or(a.ctl + kCtlError, kSchedErrXcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    scan_chunk<DK, E, NT, WC>(recb, vs + w * VC, st, ov);
  };

  // outputs of chunk ci, stored after the next barrier so their latency
  // overlaps the following chunk.  The buffer descriptor covers exactly the
  // chunk's valid rows, so rows past the end of the sequence are dropped by
  // the hardware.  The whole offset goes in the VGPR operand: the range check
  // of a raw buffer access does not include soffset.
  auto store_o = [&](int ci, f32x4 (*ov)[NT]) {
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        O + (size_t)t0 * tok_stride, 0, (int)((size_t)L * tok_stride * sizeof(E)), 0x00020000);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int o_lane = (int)(((size_t)(4 * g) * tok_stride + (size_t)h * DV + v0 + 16 * nt + col) * sizeof(E));
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row_off = (int)((size_t)(16 * I + r) * tok_stride * sizeof(E));
          // copy the lane value out of the vector first: a bit cast applied to
          // a vector-element subscript reads element 0 with this compiler
          const float x = ov[I][nt][r];
          // cache policy 2 = nontemporal: every output byte is written once
          if constexpr (sizeof(E) == 2)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f<E>(x)), rs,
                                                  o_lane + row_off, 0, 2);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), rs, o_lane + row_off, 0, 2);
        }
    }
  };

  // this wave's outputs into the LDS stage (rows 16I + 4g + r, its columns)
  auto stage_o = [&](char *ot, f32x4 (*ov)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = ov[I][nt][r];
          *reinterpret_cast<E *>(ot + (16 * I + 4 * g + r) * OROW + (w * VC + 16 * nt + col) * (int)sizeof(E)) =
              from_f<E>(x);
        }
  };

  f32x4 ov[4][NT];
  if (NBUF == 2) {
    __syncthreads();  // chunk 0 ready
    for (int ci = 0; ci < nchunks; ci += 2) {
      compute(rec0, vring[ci % NV], ov);
      stage_o(otile[ci & 1], ov);
      __syncthreads();
      if (ci + 1 >= nchunks) break;
      compute(rec1, vring[(ci + 1) % NV], ov);
      stage_o(otile[(ci + 1) & 1], ov);
      __syncthreads();
    }
  } else {
    for (int ci = 0; ci < nchunks; ++ci) {
      __syncthreads();  // buffer free
      if (ci > 0) store_o(ci - 1, ov);
      __syncthreads();  // buffer ready
      compute(rec0, vring[ci % NV], ov);
    }
    if (nchunks > 0) store_o(nchunks - 1, ov);
  }

  float *sf = a.S_final + sbase;
  if (!SCHED && a.S_last) {  // split-sequence: only the sequence's last segment
    if (n % a.seg_per_seq != a.seg_per_seq - 1) return;
    sf = a.S_last + ((size_t)(n / a.seg_per_seq) * H + h) * DV * DK + (size_t)(v0 + col) * DK;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      *reinterpret_cast<f32x4 *>(sf + (size_t)16 * nt * DK + 16 * ct + 4 * g) = st[ct][nt];
}

// ================================================= one-CU-per-unit scan
// The scan for d_k = d_v = 128 bf16 batches of many units: one workgroup per
// unit (sequence, head) on one CU instead of four, so each chunk record is
// copied into LDS once per unit, not once per 32-column group.  Its chunk
// step is longer than the four-workgroup scan's (1.9 against 1.5 us on the
// prefill shape: one CU ingests the whole record and does all 128 columns'
// products), but it holds a quarter of the CUs per unit, so it wins once the
// units outnumber the chip (more than 64 units at four workgroups each).

// One chunk for a wave owning NT 16-column tiles: the arithmetic and operand
// order of scan_chunk, with the LDS operand reads software-pipelined one step
// ahead of their products (the fragments of slab u+1 are requested before
// slab u's products, each later phase's operands before the previous phase's
// products), in fewer registers than scan_chunk's read-everything-first order,
// which three waves per SIMD cannot hold.  (Scheduling barriers that pinned
// this order exactly were measured slower: 63 against 60 us per prefill-shaped
// scan.)
template <int DK, typename E, int NT, int VSTRIDE>
__device__ __forceinline__ void scan_chunk_lean(const char *recb, const E *vs, f32x4 (*st)[NT], f32x4 (*ov)[NT]) {
  typedef RecordShape<DK, E> RS;
  typedef FragShape<E, DK> FK;   // products over d_k
  typedef FragShape<E, 64> FT;   // products over the 64 tokens
  constexpr int CT = DK / 16;
  constexpr int TILE_K = FK::NU * 64 * FK::KS;
  constexpr int TILE_T = FT::NU * 64 * FT::KS;
  const int l = lane_id(), col = l & 15, g = l >> 4;
  typedef BOps<E, DK> BK;
  typedef BOps<E, 64> BT;
  constexpr int UK = FK::NU, UT = FT::NU;
  static_assert(UT == 2, "64 tokens are two k-slabs of 32");
  const E *Kh = reinterpret_cast<const E *>(recb + RS::kh);
  const E *Qh = reinterpret_cast<const E *>(recb + RS::qh);
  const E *KtT = reinterpret_cast<const E *>(recb + RS::ktt);
  const E *Tb = reinterpret_cast<const E *>(recb + RS::tb);
  const E *Aq = reinterpret_cast<const E *>(recb + RS::aqk);
  const float *P63 = reinterpret_cast<const float *>(recb + RS::p63);
  // the (row tile, slab) fragments of a lower-triangular 64 x 64 operand, in
  // the order the products use them: slab 0 of tiles 0-3, slab 1 of tiles 2-3
  constexpr int NTRI = 6;
  auto tri_frag = [](const E *base, int f) {
    const int I = f < 4 ? f : f - 2, u = f < 4 ? 0 : 1;
    return BT::load1(base + tri_slab0(I, (int)sizeof(E)) * 64 * FT::KS, u);
  };

  // X_top = Kbnd S^T, X_bot = s Qbnd S^T, slab by slab
  typename BK::frag fk[2][4], fq[2][4];
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    fk[0][I] = BK::load1(Kh + I * TILE_K, 0);
    fq[0][I] = BK::load1(Qh + I * TILE_K, 0);
  }
  BK sb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 t[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) t[ct] = st[ct][nt];
    sb[nt].build(t);
  }
  f32x4 xt[4][NT], xb[4][NT];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) xt[I][nt] = xb[I][nt] = zero4();
#pragma unroll
  for (int u = 0; u < UK; ++u) {
    if (u + 1 < UK) {
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        fk[(u + 1) & 1][I] = BK::load1(Kh + I * TILE_K, u + 1);
        fq[(u + 1) & 1][I] = BK::load1(Qh + I * TILE_K, u + 1);
      }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        xt[I][nt] = sb[nt].mma1(fk[u & 1][I], u, xt[I][nt]);
        xb[I][nt] = sb[nt].mma1(fq[u & 1][I], u, xb[I][nt]);
      }
  }
  // E's operands and the value rows, requested behind the last X products
  typename BT::frag ftb[NTRI];
#pragma unroll
  for (int f = 0; f < NTRI; ++f) ftb[f] = tri_frag(Tb, f);
  float vv[NT][4][4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) vv[nt][I][r] = to_f(vs[(16 * I + 4 * g + r) * VSTRIDE + 16 * nt + col]);
  // Ebar = V - X_top ; E = Tb Ebar
  BT ebo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 eb[4];
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int r = 0; r < 4; ++r) eb[I][r] = vv[nt][I][r] - xt[I][nt][r];
    ebo[nt].build(eb);
  }
  typename BT::frag faq[NTRI];
#pragma unroll
  for (int f = 0; f < NTRI; ++f) faq[f] = tri_frag(Aq, f);
  f32x4 e[4][NT];
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) e[I][nt] = zero4();
#pragma unroll
  for (int f = 0; f < NTRI; ++f) {
    const int I = f < 4 ? f : f - 2, u = f < 4 ? 0 : 1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) e[I][nt] = ebo[nt].mma1(ftb[f], u, e[I][nt]);
  }
  // Kend^T, first group, requested behind E's products
  typename BT::frag fkt[2][CT / 2];
#pragma unroll
  for (int j = 0; j < CT / 2; ++j) fkt[0][j] = BT::load1(KtT + j * TILE_T, 0);
  BT eo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    f32x4 et[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) et[I] = e[I][nt];
    eo[nt].build(et);
  }
  // O = s Qbnd S^T + A E
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ov[I][nt] = xb[I][nt];
#pragma unroll
  for (int f = 0; f < NTRI; ++f) {
    const int I = f < 4 ? f : f - 2, u = f < 4 ? 0 : 1;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) ov[I][nt] = eo[nt].mma1(faq[f], u, ov[I][nt]);
  }
  // S^T = D_{0:63} S^T + Kend^T E, in four groups of four channel tiles x one
  // slab, each group's fragments requested before the previous group's
  // products issue
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const f32x4 p = *reinterpret_cast<const f32x4 *>(P63 + 16 * ct + 4 * g);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[ct][nt][r] *= p[r];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {           // group q: slab q / 2, channel tiles (q % 2) * 4 .. + 3
    const int u = q >> 1, c0 = (q & 1) * (CT / 2);
    if (q + 1 < 4) {
      const int un = (q + 1) >> 1, cn = ((q + 1) & 1) * (CT / 2);
#pragma unroll
      for (int j = 0; j < CT / 2; ++j) fkt[(q + 1) & 1][j] = BT::load1(KtT + (cn + j) * TILE_T, un);
    }
#pragma unroll
    for (int j = 0; j < CT / 2; ++j)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st[c0 + j][nt] = eo[nt].mma1(fkt[q & 1][j], u, st[c0 + j][nt]);
  }
}


// eight compute waves of 16 columns and four copy waves: measured against
// four waves of 32 columns (each fragment feeding two products, one wave per
// SIMD) and eight waves that copy as well, which were 1.3-1.7x slower
constexpr int kUnitCW = 8, kUnitCP = 4;
// The two-phase schedule takes this scan above 64 units (the four-workgroup
// scan's 256 workgroups fill the chip at 64 units; measured on the packed
// batch of 1024 units, 274,797 tokens: a call of 3412 against 3766 us).
constexpr int kUnitScanMinUnits = 64;

// The scan, one workgroup per unit: CW compute waves and CP copy waves (none:
// the compute waves issue the copies).  While the compute waves work on
// chunk c, the copiers stream chunk c+1's record (61 KiB) and value rows (64
// tokens x 128 columns) into the other half of double-buffered LDS, and touch
// chunk c+2's value rows so those come from L2, not HBM, when copied.
// Outputs go straight to o.  SCHED: the overlapped schedule (a unit per
// ticket of this XCD; a record is copied once its ready bit is set, with a
// bounded wait).
template <bool SCHED, int CW, int CP>
__global__ __launch_bounds__(64 * (CW + CP)) __attribute__((amdgpu_waves_per_eu((CW + CP + 3) / 4, (CW + CP + 3) / 4)))
void unit_scan_kernel(ScanKArgs a) {
  constexpr int DK = 128, DV = 128;
  constexpr int NT = DV / 16 / CW;               // 16-column tiles per compute wave
  constexpr int NCOPY = CP > 0 ? CP : CW;        // waves issuing copies
  typedef bf16 E;
  typedef RecordShape<DK, E> RS;
  constexpr int CT = DK / 16;
  constexpr int VROW = DV * (int)sizeof(E);      // bytes of one token's values
  constexpr int VBYTES = 64 * VROW;               // one chunk's value rows
  __shared__ __attribute__((aligned(1024))) char rec[2][RS::bytes];
  __shared__ __attribute__((aligned(1024))) char vbuf[2][VBYTES];
  __shared__ __attribute__((aligned(16))) char touch[256];

  const int w = wave_id(), l = lane_id(), col = l & 15, g = l >> 4;
  const int x = SCHED ? xcd_id() : 0;
  int u;
  if constexpr (SCHED) {
    __shared__ int sTicket;
    if (threadIdx.x == 0)
      sTicket = __hip_atomic_fetch_add(a.ctl + kCtlScanNext + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    u = x + 8 * sTicket;
  } else {
    u = blockIdx.x;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      a.ctl[kCtlSchedule] = a.sched_id ? a.sched_id : kScheduleTwoPhase;
      a.ctl[kCtlError] = 0;
    }
  }
  if (u >= a.n_units) return;
  const int n = a.seq_order ? a.seq_order[u / a.H] : u / a.H, h = u % a.H;
  const int H = a.H;
  long long tstart, ntok, chunk0;
  if (a.seq_tok0) {
    tstart = a.seq_tok0[n];
    ntok = a.seq_tok0[n + 1] - tstart;
    chunk0 = a.seq_chunk0[n];
  } else {
    tstart = (long long)n * a.T;
    ntok = a.T;
    chunk0 = (long long)n * a.nct;
  }
  const int nchunks = (int)((ntok + kChunk - 1) / kChunk);
  const E *V = reinterpret_cast<const E *>(a.v);
  E *O = reinterpret_cast<E *>(a.o);
  const size_t tok_stride = (size_t)H * DV;
  const bool copier = CP == 0 || w >= CW;
  const int cpi = CP == 0 ? w : w - CW;          // index among the copiers

  // ------------------------------------------------------------ copies
  // record: 1 KiB blocks cpi*QPW .. cpi*QPW + QPW - 1, clamped to the last
  // block (a clamped block is copied twice with the same bytes)
  auto copy_rec = [&](int ci, char *dst) {
    const char *src = a.ws_records + ((size_t)(chunk0 + ci) * H + h) * RS::bytes + l * 16;
    const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)dst;
    constexpr int NQ = RS::bytes / 1024, QPW = (NQ + NCOPY - 1) / NCOPY;
#pragma unroll
    for (int qq = 0; qq < QPW; ++qq) {
      const int q = min(cpi * QPW + qq, NQ - 1);
      lds_dma16(src + q * 1024, lds + q * 1024);
    }
  };
  // value rows: one copy moves four rows (16 lanes x 16 bytes per row); rows
  // past the end of the sequence repeat its last token (their Tb rows and
  // columns are zero, so they never reach a valid output)
  auto copy_v = [&](int ci, char *dst) {
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)dst;
    constexpr int PER = 64 / 4 / NCOPY;   // copies per copier
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) {
      const int j = cpi * PER + jj, row = 4 * j + (l >> 4);
      const E *src = V + (size_t)(t0 + min(row, L - 1)) * tok_stride + (size_t)h * DV + (l & 15) * 8;
      lds_dma16_nt(src, lds + j * 1024);
    }
  };
  // chunk ci's value rows into L2: copiers 0 and 1, one 4-byte load per
  // 128-byte line (32 rows x 2 lines each)
  const bool toucher = copier && cpi < 2;
  const uint32_t touch_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)touch;
  auto touch_v = [&](int ci) {
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const int row = 32 * cpi + (l >> 1);
    const char *src = reinterpret_cast<const char *>(V + (size_t)(t0 + min(row, L - 1)) * tok_stride +
                                                     (size_t)h * DV) + (l & 1) * 128;
    lds_dma4(src, touch_lds);
  };
  unsigned known = 0;
  int known_word = -1;
  bool gave_up = false;
  auto wait_rec = [&](int ci) {
    if constexpr (SCHED) {
      const int wd = ci >> 5;
      const unsigned bit = 1u << (ci & 31);
      if (wd != known_word) {
        known_word = wd;
        known = 0;
      }
      if ((known & bit) || gave_up) return;
      if (a.wait_ticks <= 0) {
        if (l == 0) __hip_atomic_fetch_or(a.ctl + kCtlError, kSchedErrTimeout, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        gave_up = true;
        return;
      }
      const int *word = a.ready + (size_t)u * a.ready_words + wd;
      const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        unsigned v = 0;
        if (l == 0) v = (unsigned)__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        known = __builtin_amdgcn_readfirstlane(v);
        if (known & bit) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > (unsigned long long)a.wait_ticks) {
          if (l == 0) __hip_atomic_fetch_or(a.ctl + kCtlError, kSchedErrTimeout, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
          gave_up = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
  };
  // chunk ci's copies (and the touch of chunk ci + 1's value rows, and with
  // touch_ahead of its record: copiers 2 and 3 take four 8 KiB blocks each);
  // returns the loads issued after the copies (touches, which nothing waits
  // for)
  auto issue_copies = [&](int ci) {
    if (!copier) return 0;
    wait_rec(ci);
    copy_rec(ci, rec[ci & 1]);
    copy_v(ci, vbuf[ci & 1]);
    if (ci + 1 >= nchunks) return 0;
    if (toucher) {
      touch_v(ci + 1);
      return 1;
    }
    if (!SCHED && a.touch_ahead && NCOPY == 4 && cpi >= 2) {
      touch_record<4>(a.ws_records + ((size_t)(chunk0 + ci + 1) * H + h) * RS::bytes, RS::bytes, 4 * (cpi - 2),
                      touch_lds);
      return 4;
    }
    return 0;
  };
  // this wave's copies have landed (touches issued after them may still fly)
  auto wait_copies = [&](int touched) {
    if (touched == 4) wait_vmcnt<4>();
    else if (touched) wait_vmcnt<1>();
    else wait_vmcnt<0>();
  };

  // CP > 0: chunk ci's outputs, staged by the compute waves in chunk ci's
  // value slot (row-major like the values), to o.  Copier cpi takes rows
  // 16 cpi .. 16 cpi + 15, the rows its next value copy refills, 16 bytes per
  // lane through a buffer descriptor clipped to the chunk's valid rows.
  // (Written straight from the compute waves as 2-byte stores, the outputs
  // cost 1.6 times their bytes in write traffic on the packed workload.)
  auto store_staged = [&](int ci) {
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        O + (size_t)t0 * tok_stride, 0, (int)((size_t)L * tok_stride * sizeof(E)), 0x00020000);
    constexpr int RPC = 64 / NCOPY;  // rows per copier
    f32x4 vals[RPC / 4];
#pragma unroll
    for (int jj = 0; jj < RPC / 4; ++jj) {
      const int row = RPC * cpi + 4 * jj + (l >> 4);
      vals[jj] = *reinterpret_cast<const f32x4 *>(vbuf[ci & 1] + row * VROW + (l & 15) * 16);
    }
#pragma unroll
    for (int jj = 0; jj < RPC / 4; ++jj) {
      const int row = RPC * cpi + 4 * jj + (l >> 4);
      const int off = (int)(((size_t)row * tok_stride + (size_t)h * DV) * sizeof(E)) + (l & 15) * 16;
      __builtin_amdgcn_raw_buffer_store_b128(
          __builtin_bit_cast(__attribute__((__vector_size__(16))) unsigned int, vals[jj]), rs, off, 0, 2);
    }
  };

  if constexpr (CP > 0) {
    if (copier) {
      static_assert(64 % (4 * NCOPY) == 0 && VROW == 16 * 16, "copier rows cover 16-lane row segments");
      int touched = nchunks > 0 ? issue_copies(0) : 0;
      wait_copies(touched);
      __syncthreads();  // chunk 0 ready
      for (int ci = 0; ci < nchunks; ++ci) {
        // chunk ci-1's outputs sit in the value slot the copies below refill
        // (this copier's rows); their loads into registers come first
        if (ci > 0) store_staged(ci - 1);
        touched = ci + 1 < nchunks ? issue_copies(ci + 1) : 0;
        wait_copies(touched);
        __syncthreads();  // chunk ci done and staged, chunk ci+1 ready
      }
      if (nchunks > 0) store_staged(nchunks - 1);
      __builtin_amdgcn_s_waitcnt(0);
      return;
    }
  }

  // ------------------------------------------------------------ compute
  const int v0 = w * 16 * NT;
  const size_t sbase = ((size_t)n * H + h) * DV * DK + (size_t)(v0 + col) * DK;
  f32x4 st[CT][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      st[ct][nt] = a.S0 ? *reinterpret_cast<const f32x4 *>(a.S0 + sbase + (size_t)16 * nt * DK + 16 * ct + 4 * g)
                        : zero4();

  // outputs of chunk ci straight to o: the buffer descriptor covers exactly
  // the chunk's valid rows, so rows past the end of the sequence are dropped
  // by the hardware (the whole offset goes in the VGPR operand: the range
  // check of a raw buffer access does not include soffset); nontemporal
  auto store_o = [&](int ci, f32x4 (*ov)[NT]) {
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        O + (size_t)t0 * tok_stride, 0, (int)((size_t)L * tok_stride * sizeof(E)), 0x00020000);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int o_lane = (int)(((size_t)(4 * g) * tok_stride + (size_t)h * DV + v0 + 16 * nt + col) * sizeof(E));
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row_off = (int)((size_t)(16 * I + r) * tok_stride * sizeof(E));
          const float xv = ov[I][nt][r];  // copied out of the vector before the bit cast
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f<E>(xv)), rs,
                                                o_lane + row_off, 0, 2);
        }
    }
  };

  int touched = (CP == 0 && nchunks > 0) ? issue_copies(0) : 0;
  if (CP == 0) wait_copies(touched);
  __syncthreads();  // chunk 0 ready
  f32x4 ov[4][NT];
  for (int ci = 0; ci < nchunks; ++ci) {
    // buffers (ci+1) % 2 held chunk ci-1, finished before the last barrier
    touched = (CP == 0 && ci + 1 < nchunks) ? issue_copies(ci + 1) : 0;
    const char *recb = rec[ci & 1];
    if constexpr (SCHED) {
      // the record must come from this XCD's prep workers (stamped by them)
      static_assert(RS::p63 + DK * 4 + 4 <= RS::bytes, "room for the XCD stamp");
      if (w == 0 && l == 0 && *reinterpret_cast<const int *>(recb + RS::p63 + DK * 4) != x)
        __hip_atomic_fetch_or(a.ctl + kCtlError, kSchedErrXcd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    scan_chunk_lean<DK, E, NT, DV>(recb, reinterpret_cast<const E *>(vbuf[ci & 1]) + v0, st, ov);
    if constexpr (CP > 0) {
      // into this chunk's value slot, over this wave's own columns (which
      // only this wave read)
      E *ot = reinterpret_cast<E *>(vbuf[ci & 1]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int I = 0; I < 4; ++I)
#pragma unroll
          for (int r = 0; r < 4; ++r) ot[(16 * I + 4 * g + r) * DV + v0 + 16 * nt + col] = from_f<E>(ov[I][nt][r]);
    } else {
      store_o(ci, ov);
    }
    if (CP == 0) wait_copies(touched);
    __syncthreads();  // chunk ci done, chunk ci+1 ready
  }
  float *sf = a.S_final + sbase;
  if (!SCHED && a.S_last) {  // split-sequence: only the sequence's last segment
    if (n % a.seg_per_seq != a.seg_per_seq - 1) return;
    sf = a.S_last + ((size_t)(n / a.seg_per_seq) * H + h) * DV * DK + (size_t)(v0 + col) * DK;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      *reinterpret_cast<f32x4 *>(sf + (size_t)16 * nt * DK + 16 * ct + 4 * g) = st[ct][nt];
}

// ======================================================= output norm + gate
// One pass over o after the scan (kda_module_ops): per token and head,
//   o <- o / sqrt(mean_c o_c^2 + eps) * w   (RMS norm over the d_v values, with
//                                            gains w; when w is given)
//   o <- o * sigmoid(g)                     (g the gate logits; when given)
// in fp32, rounded to E once.  LPR lanes per (token, head) row, 16 bytes of
// it each, and kNormRows rows per lane group, kThreads / LPR rows apart, all
// requested before any is used (on the prefill workload's 50 MB: 18.5 us with
// four rows, 19.6 with one, 19.4 with eight); tokens [tok_begin, tok_end), from
// the sequence offsets when seq_tok0 is given (a packed batch: rows outside
// every sequence are left alone), else [0, n_tok).
constexpr int kNormRows = 4;
template <typename E, int LPR>
__global__ __launch_bounds__(kThreads) void out_norm_gate_kernel(void *o, const void *gate, const float *w, float eps,
                                                                int H, long long n_tok, const int32_t *seq_tok0,
                                                                int n_seq) {
  typedef typename Row16<E>::vec RV;
  constexpr int VE = Row16<E>::N, DV = LPR * VE, GR = kThreads / LPR;
  const int part = threadIdx.x % LPR;
  long long tb = 0, te = n_tok;
  if (seq_tok0) {
    tb = seq_tok0[0];
    te = seq_tok0[n_seq];
  }
  // rows (token * H + head) of this lane group; a group's lanes share them, so
  // the sums below stay within groups whose rows are all valid or all not
  const long long row0 = tb * H + (long long)blockIdx.x * GR * kNormRows + threadIdx.x / LPR, rend = te * H;
  E *const po = reinterpret_cast<E *>(o) + part * VE;
  const E *const pg = reinterpret_cast<const E *>(gate) + part * VE;
  RV x[kNormRows], gv[kNormRows];
#pragma unroll
  for (int i = 0; i < kNormRows; ++i) {
    const long long row = row0 + (long long)i * GR;
    if (row < rend) {
      x[i] = __builtin_nontemporal_load(reinterpret_cast<const RV *>(po + (size_t)row * DV));
      if (gate) gv[i] = __builtin_nontemporal_load(reinterpret_cast<const RV *>(pg + (size_t)row * DV));
    }
  }
  f32x4 g4[VE / 4];
  if (w) {
#pragma unroll
    for (int j = 0; j < VE; j += 4) g4[j / 4] = *reinterpret_cast<const f32x4 *>(w + part * VE + j);
  }
#pragma unroll
  for (int i = 0; i < kNormRows; ++i) {
    const long long row = row0 + (long long)i * GR;
    if (row >= rend) break;  // later rows are further out
    float y[VE];
#pragma unroll
    for (int j = 0; j < VE; ++j) y[j] = (float)x[i][j];
    if (w) {
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < VE; ++j) ss += y[j] * y[j];
      const float rn = __builtin_amdgcn_rsqf(group_sum<LPR>(ss) * (1.f / DV) + eps);
#pragma unroll
      for (int j = 0; j < VE; ++j) y[j] = y[j] * rn * g4[j / 4][j % 4];
    }
    if (gate) {
#pragma unroll
      for (int j = 0; j < VE; ++j) y[j] *= sigmoid_f((float)gv[i][j]);
    }
    RV out;
#pragma unroll
    for (int j = 0; j < VE; ++j) out[j] = (E)y[j];
    __builtin_nontemporal_store(out, reinterpret_cast<RV *>(po + (size_t)row * DV));
  }
}

// The norm and gate pass over n_tok x H rows (n_tok: an upper bound when
// seq_tok0 gives the rows' range).
template <typename E>
hipError_t launch_norm_gate_rows(void *o, const void *gate, const float *w, float eps, int H, long long n_tok, int dv,
                                 const int32_t *seq_tok0, int n_seq, hipStream_t stream) {
  if (!w && !gate) return hipSuccess;
  constexpr int VE = Row16<E>::N;
  const int lpr = dv / VE;
  const long long rows = n_tok * H;
  if (rows == 0) return hipSuccess;
  const long long groups = (rows + kNormRows - 1) / kNormRows;  // lane groups of kNormRows rows
  const dim3 grid((unsigned)((groups * lpr + kThreads - 1) / kThreads));
#define KDA_POST(L)                                                                                            \
  case L:                                                                                                      \
    hipLaunchKernelGGL((out_norm_gate_kernel<E, L>), grid, dim3(kThreads), 0, stream, o, gate, w, eps, H, n_tok, \
                       seq_tok0, n_seq);                                                                       \
    break;
  switch (lpr) {
    KDA_POST(2)
    KDA_POST(4)
    KDA_POST(8)
    KDA_POST(16)
    KDA_POST(32)
    default: return hipErrorInvalidValue;
  }
#undef KDA_POST
  return hipGetLastError();
}

template <typename E>
hipError_t launch_out_post(const PrefillArgs &a, const int32_t *seq_tok0, hipStream_t stream) {
  const long long n_tok = seq_tok0 ? a.T : (long long)a.B * a.T;
  return launch_norm_gate_rows<E>(a.o, a.out_gate, a.norm_w, a.norm_eps, a.H, n_tok, a.dv, seq_tok0, a.plan.n_seq,
                                  stream);
}

// The convolution state at the end of a prefill (kda_module_ops.conv_state):
// the last three raw tokens of each (sequence, head), oldest first, q | k | v
// per token, zeros for positions before the sequence's first token.  One
// workgroup per unit; sequences from the packed tables when given.
template <typename E>
__global__ __launch_bounds__(256) void conv_state_kernel(const E *q, const E *k, const E *v, E *cs, int H, int dk,
                                                         int dv, int T, const int32_t *seq_tok0, int n_units) {
  const int unit = blockIdx.x;
  if (unit >= n_units) return;
  const int n = unit / H, h = unit % H, W = 2 * dk + dv;
  long long tb = (long long)n * T, te = tb + T;
  if (seq_tok0) {
    tb = seq_tok0[n];
    te = seq_tok0[n + 1];
  }
  E *out = cs + (size_t)unit * 3 * W;
  for (int i = threadIdx.x; i < 3 * W; i += blockDim.x) {
    const int slot = i / W, c = i % W;
    const long long t = te - 3 + slot;
    E x = (E)0.f;
    if (t >= tb) {
      const size_t th = (size_t)t * H + h;
      x = c < dk ? q[th * dk + c] : (c < 2 * dk ? k[th * dk + c - dk] : v[th * dv + c - 2 * dk]);
    }
    out[i] = x;
  }
}

// Zeroes the control words and the ready words of the overlapped schedule
// and records that schedule as the one this call runs.
__global__ void sched_clear_kernel(int *ctl, int *ready, int n_ready) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  if (tid < kCtlWords) ctl[tid] = tid == kCtlSchedule ? kScheduleOverlap : 0;
  for (int i = tid; i < n_ready; i += gridDim.x * blockDim.x) ready[i] = 0;
}

// The prep kernel for a gate form, with or without the q, k activation (and
// the convolution).
template <int DK, typename E, bool ACTQK, bool SCHED = false, bool CONV = false>
void launch_prep(int gate, dim3 grid, hipStream_t stream, const PrepKArgs &pa) {
#define KDA_PREP_LAUNCH(G)                                                                                         \
  if constexpr (CONV)                                                                                              \
    hipLaunchKernelGGL((chunk_prep_conv_kernel<DK, E, G>), grid, dim3(kThreads), 0, stream, pa);                   \
  else                                                                                                             \
    hipLaunchKernelGGL((chunk_prep_kernel<DK, E, G, ACTQK, SCHED>), grid, dim3(kThreads), 0, stream, pa);
  switch (gate) {
    case kGateScalar: KDA_PREP_LAUNCH(kGateScalar) break;
    case kGateNone: KDA_PREP_LAUNCH(kGateNone) break;
    case kGateLogChannel: KDA_PREP_LAUNCH(kGateLogChannel) break;
    case kGateLogScalar: KDA_PREP_LAUNCH(kGateLogScalar) break;
    case kGateSoftplusChannel: KDA_PREP_LAUNCH(kGateSoftplusChannel) break;
    case kGateSoftplusScalar: KDA_PREP_LAUNCH(kGateSoftplusScalar) break;
    default: KDA_PREP_LAUNCH(kGateChannel)
  }
#undef KDA_PREP_LAUNCH
}

// LDS held by one stage (record + value slices) of a scan configuration.
template <int DK, typename E> constexpr bool scan_stage_fits(int nt, int cw) {
  return RecordShape<DK, E>::bytes + cw * 64 * 16 * nt * (int)sizeof(E) <= 160 * 1024 - 1024;
}

template <int DK, typename E, int NT, int NCP>
void launch_scan(int cw, dim3 grid, hipStream_t stream, const ScanKArgs &sa) {
  if constexpr (scan_stage_fits<DK, E>(NT, 2))
    if (cw == 2) {
      hipLaunchKernelGGL((chunk_scan_kernel<DK, E, NT, 2, NCP>), grid, dim3(64 * (2 + NCP)), 0, stream, sa);
      return;
    }
  hipLaunchKernelGGL((chunk_scan_kernel<DK, E, NT, 1, NCP>), grid, dim3(64 * (1 + NCP)), 0, stream, sa);
}

// ================================================== split-sequence prefill
// A dense batch of few long sequences leaves most of the chip idle in the
// scan, whose chain is as long as a sequence's chunk count.  The step from
// one chunk's start state to the next is affine in the state (in the scan's
// terms S^T <- (D_{0:63} - Kend^T Tb Kbnd) S^T + Kend^T Tb V), so the map over
// a segment of chunks is S_end = S_start M + X: X the segment's scan from
// S = 0, M^T the scan of the d_k columns of the identity with V = 0.  The
// maps of all segments but the last run at once (map_scan_kernel), a small
// pass chains them into every segment's start state (split_chain_kernel),
// and the scan then runs all segments at once from those states.

struct MapKArgs {
  const void *v;
  const char *ws_records;
  float *maps;          // per map unit (sequence, segment < G-1, head): X rows (d_v), then M^T rows (d_k), fp32 x d_k
  int H, T, nct;        // dense batch: sequences of T tokens, nct chunks
  int G, cps;           // segments per sequence, chunks per segment
  int n_maps;           // B (G - 1) H
  int touch_ahead;      // pull record ci+2 into L2 while chunk ci runs
};

// One workgroup per (map unit, group of 16 CW columns): the groups
// 0 .. DV/WC-1 scan value columns from S = 0 (X), the rest scan columns of the
// identity with V = 0 (M^T).  The state update alone (scan_chunk without
// outputs), so only Kbnd, Kend^T, Tb and D_{0:63} of each record are copied.
// Workgroups of one map unit get ids congruent mod 8 (one XCD).
template <int CW, int NCP>
__global__ __launch_bounds__(64 * (CW + NCP)) __attribute__((amdgpu_waves_per_eu(1, 1)))
void map_scan_kernel(MapKArgs a) {
  constexpr int DK = 128, DV = 128;
  typedef bf16 E;
  typedef RecordShape<DK, E> RS;
  constexpr int CT = DK / 16;
  constexpr int WC = CW * 16;                // columns per workgroup
  constexpr int GX = DV / WC, GM = DK / WC;  // workgroups per map unit: X columns, M columns
  __shared__ __attribute__((aligned(1024))) char rec[2][RS::bytes];
  __shared__ __attribute__((aligned(1024))) E vt[2][64 * WC];
  __shared__ __attribute__((aligned(16))) char touch_area[256];

  const int w = wave_id(), l = lane_id(), col = l & 15, g = l >> 4;
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int mu = (slot / (GX + GM)) * 8 + xcd, grp = slot % (GX + GM);
  if (mu >= a.n_maps) return;
  const int nm = mu / a.H, h = mu % a.H;
  const int n = nm / (a.G - 1), sg = nm % (a.G - 1);
  const long long tstart = (long long)n * a.T + (long long)sg * a.cps * kChunk;
  const long long chunk0 = (long long)n * a.nct + (long long)sg * a.cps;
  const int nchunks = a.cps;  // segments before the last are whole chunks
  const bool ident = grp >= GX;
  const int c0 = (ident ? grp - GX : grp) * WC;  // first value column / identity column
  const E *V = reinterpret_cast<const E *>(a.v);
  const size_t tok_stride = (size_t)a.H * DV;

  if (w >= CW) {
    const int cpi = w - CW;
    // 1 KiB blocks of Kbnd, of Kend^T and Tb (adjacent), and of D_{0:63}
    constexpr int B_KH = RS::kh / 1024, N_KH = (RS::qh - RS::kh) / 1024;
    constexpr int B_KT = RS::ktt / 1024, N_KT = (RS::aqk - RS::ktt) / 1024;
    constexpr int B_P = RS::p63 / 1024, N_P = (RS::bytes - RS::p63) / 1024;
    constexpr int NB = N_KH + N_KT + N_P, QPW = (NB + NCP - 1) / NCP;
    static_assert(RS::kh % 1024 == 0 && RS::ktt % 1024 == 0 && RS::aqk % 1024 == 0 && RS::p63 % 1024 == 0,
                  "record parts on 1 KiB boundaries");
    auto copy_rec = [&](int ci, char *dst) {
      const char *src = a.ws_records + ((size_t)(chunk0 + ci) * a.H + h) * RS::bytes + l * 16;
      const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)dst;
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        const int b = min(cpi * QPW + qq, NB - 1);  // clamped blocks are copied twice, same bytes
        const int blk = b < N_KH ? B_KH + b : (b < N_KH + N_KT ? B_KT + b - N_KH : B_P + b - N_KH - N_KT);
        lds_dma16(src + blk * 1024, lds + blk * 1024);
      }
    };
    // the value columns c0 .. c0+WC-1 of chunk ci: 64 rows of WC elements,
    // 1 KiB per copy
    constexpr int LPR = WC * (int)sizeof(E) / 16, RPI = 64 / LPR;
    auto copy_v = [&](int ci, E *dst) {
      const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) E *)dst;
#pragma unroll
      for (int j = 0; j < 64 / RPI; ++j) {
        const E *src = V + (size_t)(tstart + (long long)kChunk * ci + j * RPI + l / LPR) * tok_stride +
                       (size_t)h * DV + c0 + (l % LPR) * (16 / (int)sizeof(E));
        lds_dma16_nt(src, lds + j * 1024);
      }
    };
    const bool vcopier = !ident && cpi == NCP - 1;
    const uint32_t touch_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)touch_area;
    if (nchunks > 0) {
      copy_rec(0, rec[0]);
      if (vcopier) copy_v(0, vt[0]);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // chunk 0 ready
    for (int ci = 0; ci < nchunks; ++ci) {
      // buffers (ci+1)%2 held chunk ci-1, finished before the last barrier
      if (ci + 1 < nchunks) {
        copy_rec(ci + 1, rec[(ci + 1) & 1]);
        if (vcopier) copy_v(ci + 1, vt[(ci + 1) & 1]);
      }
      if (a.touch_ahead && cpi == 1 && !vcopier && ci + 2 < nchunks) {
        // record ci+2 into L2: this workgroup's share of its eight 8 KiB blocks
        constexpr int TB = 8 / (GX + GM);
        touch_record<TB>(a.ws_records + ((size_t)(chunk0 + ci + 2) * a.H + h) * RS::bytes, RS::bytes, TB * grp,
                         touch_lds);
        wait_vmcnt<TB>();  // the copies; the touches may still fly
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __syncthreads();  // chunk ci done, chunk ci+1 ready
    }
    __builtin_amdgcn_s_waitcnt(0);
    return;
  }

  // compute waves: S^T (d_k x 16 columns) in accumulator tiles, from 0 or
  // from the identity's columns v0 .. v0+15
  const int v0 = c0 + w * 16;
  f32x4 st[CT][1], ov[4][1];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) st[ct][0][r] = ident && 16 * ct + 4 * g + r == v0 + col ? 1.f : 0.f;
  __syncthreads();  // chunk 0 ready
  for (int ci = 0; ci < nchunks; ++ci) {
    if (ident)
      scan_chunk<DK, E, 1, WC, false, true>(rec[ci & 1], nullptr, st, ov);
    else
      scan_chunk<DK, E, 1, WC, false, false>(rec[ci & 1], vt[ci & 1] + w * 16, st, ov);
    __syncthreads();
  }
  float *out = a.maps + (size_t)mu * (DV + DK) * DK + (size_t)((ident ? DV : 0) + v0 + col) * DK;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) *reinterpret_cast<f32x4 *>(out + 16 * ct + 4 * g) = st[ct][0];
}

// Segment tables in the packed-batch form the scan reads: segment i = n G + g
// starts at token n T + min(g cps 64, T) and at chunk slot n nct + g cps
// (written by the chain pass's first workgroup; the scan runs after it).
struct SplitTables {
  int32_t *tok0, *chunk0;
  int B, T, nct, cps;
};
__device__ __forceinline__ void write_split_tables(const SplitTables &tb, int G) {
  for (int i = threadIdx.x; i <= tb.B * G; i += blockDim.x) {
    const int n = i / G, sg = i % G;
    tb.tok0[i] = (int32_t)((long long)n * tb.T + min((long long)sg * tb.cps * kChunk, (long long)tb.T));
    tb.chunk0[i] = (int32_t)((long long)n * tb.nct + (long long)sg * tb.cps);
  }
}

// Segment start states: S_0 = S0 (or zero), S_{g+1} = S_g M_g + X_g in fp32
// (S-form, d_v x d_k; M_g's rows are the stored M^T rows, so the product is
// sum_j S_g[r][j] Mt_g[j][c]).  Rows are independent: one workgroup per
// (sequence, head, block of RB = 4 rows); start is [B G H] x d_v x d_k.
// Wave q takes the key channels j in [32 q, 32 q + 32) of the product and
// lane c the columns 2c and 2c + 1: those 32 x 2 entries of Mt stay in the
// lane's registers, loaded a segment ahead (one contiguous 512-byte row per
// wave and load), the four rows of S_g are read from LDS as wave-wide
// broadcasts, and the four waves' partial sums meet in LDS, where thread
// (row q, columns 2c, 2c + 1) adds them to X_g.  Measured on 4 heads x 16
// segments: 1.7 us per segment (the kernel 38 us), against about 3 us (49) for
// the earlier form with all of Mt in LDS and a thread per row and column
// pair, bound by its 256 KiB of LDS reads.  The bound now is moving Mt, 64
// KiB per workgroup and segment: without those loads (results wrong, timing
// only) a segment took 0.9 us, and loading Mt two segments ahead, or in eight
// parts between the steps of the product, changed nothing.
template <int RB>
__global__ __launch_bounds__(256) void split_chain_kernel(const float *S0, const float *maps, float *start, int H,
                                                          int G, int n_units, SplitTables tb) {
  if (blockIdx.x == 0) write_split_tables(tb, G);
  constexpr int DK = 128, DV = 128, JQ = DK / 4;  // key channels per wave
  static_assert(RB == 4, "four rows per workgroup: one per wave in the sums");
  typedef float f2 __attribute__((ext_vector_type(2)));
  __shared__ __attribute__((aligned(16))) float sS[RB][DK];
  __shared__ __attribute__((aligned(16))) f2 sP[4][RB][64];  // partial sums: wave, row, column pair
  const int unit = blockIdx.x / (DV / RB), rb = blockIdx.x % (DV / RB);
  if (unit >= n_units) return;  // whole workgroup
  const int n = unit / H, h = unit % H;
  // product: wave q's channels, lane c's columns; sums: row q, the same columns
  const int q = threadIdx.x >> 6, c = threadIdx.x & 63, cc = 2 * c;
  auto seg_maps = [&](int sg) { return maps + (((size_t)n * (G - 1) + sg) * H + h) * (size_t)(DV + DK) * DK; };
  auto start_row = [&](int sg) {
    return start + (((size_t)n * G + sg) * H + h) * DV * DK + (size_t)(rb * RB + q) * DK + cc;
  };
  {
    f2 x = {0.f, 0.f};
    if (S0) x = *reinterpret_cast<const f2 *>(S0 + ((size_t)unit * DV + rb * RB + q) * DK + cc);
    *reinterpret_cast<f2 *>(&sS[q][cc]) = x;
    *reinterpret_cast<f2 *>(start_row(0)) = x;
  }
  // Mt_sg's rows 32 q .. 32 q + 31 at columns cc, cc + 1, and X_sg's entries of this thread's sum
  auto load_map = [&](int sg, f2 *m, f2 &x) {
    x = *reinterpret_cast<const f2 *>(seg_maps(sg) + (size_t)(rb * RB + q) * DK + cc);
    const float *Mt = seg_maps(sg) + (size_t)DV * DK + (size_t)(JQ * q) * DK + cc;
#pragma unroll
    for (int jj = 0; jj < JQ; ++jj) m[jj] = *reinterpret_cast<const f2 *>(Mt + (size_t)jj * DK);
  };
  // one segment with the map in (m, x), the next one's loads into (mn, xn)
  auto hop = [&](int sg, const f2 *m, const f2 x, f2 *mn, f2 &xn) {
    __syncthreads();  // S_sg complete in sS
    // the next segment's map, in flight during the product (the last
    // segment reloads its own: every segment issues the same loads, so the
    // waits for this segment's map can leave the next one's in flight)
    load_map(sg + 2 < G ? sg + 1 : sg, mn, xn);
    __builtin_amdgcn_sched_barrier(0);  // issued before the product, not sunk below it
    f2 acc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) acc[r] = f2{0.f, 0.f};
#pragma unroll
    for (int j4 = 0; j4 < JQ; j4 += 4) {
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        const f32x4 s4 = *reinterpret_cast<const f32x4 *>(&sS[r][JQ * q + j4]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          acc[r].x = __builtin_fmaf(s4[jj], m[j4 + jj].x, acc[r].x);
          acc[r].y = __builtin_fmaf(s4[jj], m[j4 + jj].y, acc[r].y);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) sP[q][r][c] = acc[r];
    __syncthreads();  // partial sums complete, and every wave is done reading S_sg
    f2 y = x;
#pragma unroll
    for (int w = 0; w < 4; ++w) y += sP[w][q][c];
    *reinterpret_cast<f2 *>(&sS[q][cc]) = y;
    *reinterpret_cast<f2 *>(start_row(sg + 1)) = y;
  };
  f2 mA[JQ], mB[JQ], xA, xB;
  if (G > 1) load_map(0, mA, xA);
  for (int sg = 0; sg + 1 < G; sg += 2) {
    hop(sg, mA, xA, mB, xB);
    if (sg + 2 < G) hop(sg + 1, mB, xB, mA, xA);
  }
}



// ================================================================ dispatch
// CU-masked streams of the overlapped schedule, one set per device: the scan
// on the first 128 CUs of the runtime's mask numbering (16 per XCD) and the
// prep on the next 112 (14 per XCD), so neither can hold the CUs the other
// needs.  The last 16 CUs stay idle: on a 1024-chunk chain the prep, which
// finishes well before the scan, slowed the scan less on 112 CUs (a call of
// 1833-1839 us) than on 128 (1985 us) or 96 (1852 us); on 80 it became the
// bound (2441 us).
// Created on the first overlapped call on a device; released by
// kda_release() (also run at process exit, before the HIP runtime and any
// profiler attached to it are torn down: streams still alive at that point
// were destroyed by the runtime's own teardown after the profiler had
// finalised, and the process then crashed in __cxa_finalize).
struct OverlapCtx {
  bool tried = false, ok = false;
  hipStream_t scan = nullptr, prep = nullptr;
  hipEvent_t fork = nullptr, done_scan = nullptr, done_prep = nullptr;
};
std::mutex g_overlap_mu;  // guards g_overlap and the event sequence of a launch
OverlapCtx g_overlap[64];
bool g_atexit_registered = false;  // guarded by g_overlap_mu
constexpr int kScanCUs = 128, kPrepCUs = 112;
// copy waves of the overlapped scan: four measured 4 % faster than three on
// a 1024-chunk chain
constexpr int kOverlapCopyWaves = 4;

// Destroys what one device's context holds (caller holds g_overlap_mu and
// has made that device current).
void destroy_ctx(OverlapCtx &c) {
  if (c.scan) (void)hipStreamDestroy(c.scan);
  if (c.prep) (void)hipStreamDestroy(c.prep);
  if (c.fork) (void)hipEventDestroy(c.fork);
  if (c.done_scan) (void)hipEventDestroy(c.done_scan);
  if (c.done_prep) (void)hipEventDestroy(c.done_prep);
  c = OverlapCtx{};
}

void release_at_exit() { release_overlap(); }

// The current device's streams, or null if the schedule cannot run there
// (caller holds g_overlap_mu).  A call whose stream is being captured into a
// graph never takes the overlapped schedule: a graph replay keeps neither
// the compute-unit masks nor the guarantee that the prep runs beside the
// scan, whose waits would then time out.
OverlapCtx *overlap_ctx(hipStream_t stream) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  OverlapCtx &c = g_overlap[dev];
  if (!c.tried) {
    c.tried = true;
    int ncu = 0;
    hipDeviceProp_t prop;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return nullptr;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return nullptr;
    // eight XCDs of 32 CUs (the whole MI355X as one device)
    if (ncu != 256 || std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return nullptr;
    if (!g_atexit_registered) g_atexit_registered = std::atexit(release_at_exit) == 0;
    uint32_t ms[8] = {0}, mp[8] = {0};
    for (int i = 0; i < kScanCUs + kPrepCUs; ++i) (i < kScanCUs ? ms : mp)[i / 32] |= 1u << (i % 32);
    if (hipExtStreamCreateWithCUMask(&c.scan, 8, ms) != hipSuccess ||
        hipExtStreamCreateWithCUMask(&c.prep, 8, mp) != hipSuccess ||
        hipEventCreateWithFlags(&c.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c.done_scan, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c.done_prep, hipEventDisableTiming) != hipSuccess) {
      destroy_ctx(c);
      c.tried = true;  // stay on two-phase on this device
      return nullptr;
    }
    c.ok = true;
  }
  return c.ok ? &c : nullptr;
}

// Shapes the overlapped schedule supports: dense bf16 batches at
// d_k = d_v = 128 (two records and two value tiles fill the scan's LDS).
// Not with the short convolution, whose prep writes the convolved v that the
// scan reads.
template <int DK, typename E> bool overlap_supported(const PrefillArgs &a) {
  return DK == 128 && a.dv == 128 && sizeof(E) == 2 && !a.cu_seqlens && a.plan.ready_bytes > 0 && !a.conv_q;
}

// Automatic choice: the overlap needs the scan's workgroups (four per unit at
// d_v = 128) to fit on its 128 CUs, and it pays once the batch holds at least
// 4096 chunk records (256 MB at d = 128, the size of the Infinity Cache):
// the two-phase scan then fetches its records from HBM while the overlapped
// one reads them soon after they are written, and the fork and join of the
// two streams (about 24 us, measured with empty kernels) are amortised.
// Measured (two-phase / overlap, us): 8 units x 256 chunks 300 / 380, 8 x 512
// 800 / 759, 16 x 192 293 / 336, 16 x 256 477 / 419, 32 x 128 310 / 315,
// 32 x 192 473 / 416, 32 x 1024 2430 / 1800.
constexpr long long kOverlapMinRecords = 4096;
bool overlap_chosen(const PrefillArgs &a, int nct) {
  if (a.schedule == kScheduleTwoPhase) return false;
  if (a.schedule == kScheduleOverlap) return true;
  const long long units = (long long)a.B * a.H;
  return units * (a.dv / 32) <= kScanCUs && units * nct >= kOverlapMinRecords;
}

// Overlapped schedule: clear the ready words on the caller's stream, then
// fork to the two masked streams (the scan and the prep run at once, the
// scan's copy waves waiting on each record's ready bit), and join back.
template <int DK, typename E>
hipError_t run_prefill_overlap(const PrefillArgs &a, hipStream_t stream, PrepKArgs pa, const ChunkRecordLayout &lay,
                               char *records, OverlapCtx &ov) {
  const WorkspacePlan &P = a.plan;
  const int nct = (a.T + kChunk - 1) / kChunk;
  const int n_units = a.B * a.H;
  const int words = (nct + 31) / 32;  // ready words per unit
  int *ready = reinterpret_cast<int *>(a.ws + P.ready);  // n_units * words <= chunk slots * heads
  int *ctl = reinterpret_cast<int *>(a.ws);
  const int nclear = (int)(P.max_chunks * a.H);
  hipLaunchKernelGGL(sched_clear_kernel, dim3((unsigned)min(64, (nclear + 255) / 256)), dim3(256), 0, stream, ctl,
                     ready, nclear);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(ov.fork, stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(ov.scan, ov.fork, 0)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(ov.prep, ov.fork, 0)) != hipSuccess) return e;

  if constexpr (DK == 128 && sizeof(E) == 2) {
    ScanKArgs sa{};
    sa.v = a.v;
    sa.S0 = a.S0;
    sa.o = a.o;
    sa.S_final = a.S_final;
    sa.ws_records = records;
    sa.lay = lay;
    sa.H = a.H;
    sa.dv = a.dv;
    sa.T = a.T;
    sa.nct = nct;
    sa.seq_tok0 = sa.seq_chunk0 = sa.seq_order = nullptr;
    sa.scale = a.scale;
    sa.n_units = n_units;
    sa.wg_per_unit = a.dv / 32;  // two compute waves of 16 columns per workgroup
    sa.ready = ready;
    sa.ready_words = words;
    sa.ctl = ctl;
    sa.wait_ticks = a.wait_ticks;
    // a ticket per (unit, group): eight times those of the XCD with most units
    const dim3 sg((unsigned)(8 * ((n_units + 7) / 8) * sa.wg_per_unit));
    hipLaunchKernelGGL((chunk_scan_kernel<DK, E, 1, 2, kOverlapCopyWaves, true>), sg, dim3(64 * (2 + kOverlapCopyWaves)),
                       0, ov.scan, sa);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    pa.ready = ready;
    pa.ctl = ctl;
    pa.ready_words = words;
    pa.n_units = n_units;
    // one workgroup per task: eight times the task count of the XCD with most units
    const dim3 pg((unsigned)(8LL * ((n_units + 7) / 8) * nct));
    if (a.act & kActQK)
      launch_prep<DK, E, true, true>(a.gate, pg, ov.prep, pa);
    else
      launch_prep<DK, E, false, true>(a.gate, pg, ov.prep, pa);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = hipEventRecord(ov.done_scan, ov.scan)) != hipSuccess) return e;
  if ((e = hipEventRecord(ov.done_prep, ov.prep)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(stream, ov.done_scan, 0)) != hipSuccess) return e;
  return hipStreamWaitEvent(stream, ov.done_prep, 0);
}

// The two-phase scan over sa.n_units units (sa filled in but for the
// workgroup shape).  Two compute waves of one 16-column tile each per
// workgroup (one wave when d_v = 16 or two stages would not fit in LDS) and
// four copy waves: measured fastest at d_v = 128 against two tiles per wave
// (which halves the LDS reads per column but doubles each wave's serial chain
// of products) and against one, two, three, five and six copy waves.  Past 64
// units at d = 128 bf16, one workgroup per unit.
template <int DK, typename E>
hipError_t launch_scan_phase(const PrefillArgs &a, ScanKArgs sa, hipStream_t stream) {
  if (DK == 128 && sizeof(E) == 2 && a.dv == 128 && sa.n_units > kUnitScanMinUnits) {
    // one workgroup per unit (units in dispatch order: longest packed
    // sequences first)
    sa.wg_per_unit = 1;
    hipLaunchKernelGGL((unit_scan_kernel<false, kUnitCW, kUnitCP>), dim3((unsigned)sa.n_units),
                       dim3(64 * (kUnitCW + kUnitCP)), 0, stream, sa);
  } else {
    int cw = a.dv >= 32 ? 2 : 1;
    while (cw > 1 && !scan_stage_fits<DK, E>(1, cw)) cw /= 2;
    sa.wg_per_unit = a.dv / (16 * cw);
    const long long slots = ((long long)sa.n_units + 7) / 8 * 8 * sa.wg_per_unit;
    launch_scan<DK, E, 1, 4>(cw, dim3((unsigned)slots), stream, sa);
  }
  return hipGetLastError();
}

// Split-sequence schedule after the prep (d = 128 bf16, dense): the maps of
// all segments but the last, the chained start states (and the segment
// tables), the scan of every segment, and the final states.
template <int DK, typename E>
hipError_t run_split(const PrefillArgs &a, hipStream_t stream, char *records, const ChunkRecordLayout &lay) {
  const WorkspacePlan &P = a.plan;
  const int G = P.split.G, cps = P.split.cps, nct = (a.T + kChunk - 1) / kChunk;
  int32_t *tok0 = reinterpret_cast<int32_t *>(a.ws + P.sp_tables);
  int32_t *ch0 = tok0 + ((size_t)a.B * G + 1);
  float *maps = reinterpret_cast<float *>(a.ws + P.sp_maps);
  float *start = reinterpret_cast<float *>(a.ws + P.sp_start);
  float *end = reinterpret_cast<float *>(a.ws + P.sp_end);
  int *ctl = reinterpret_cast<int *>(a.ws);
  const bool touch = (size_t)P.max_chunks * a.H * lay.bytes > ((size_t)256 << 20);
  const void *vsrc = a.conv_q ? a.o : a.v;  // the prep left v's convolution in o
  hipError_t e = hipSuccess;

  MapKArgs ma{};
  ma.v = vsrc;
  ma.ws_records = records;
  ma.maps = maps;
  ma.H = a.H;
  ma.T = a.T;
  ma.nct = nct;
  ma.G = G;
  ma.cps = cps;
  ma.n_maps = a.B * (G - 1) * a.H;
  ma.touch_ahead = touch;
  // two or four compute waves per workgroup, as the plan chose (measured
  // with records from the Infinity Cache, 4 heads x 16 segments: 480
  // two-wave workgroups in two rounds 140 us, 240 four-wave ones in one
  // round 91 us; 16 heads x 4 segments: 256 two-wave workgroups 384 us,
  // 128 four-wave ones 485 us)
  constexpr int kMapCP = 4;
  const int map_cw = P.split.map_cw == 4 ? 4 : 2;
  const dim3 mg((unsigned)((ma.n_maps + 7) / 8 * 8 * ((128 + 128) / (16 * map_cw))));
  if (map_cw == 4)
    hipLaunchKernelGGL((map_scan_kernel<4, kMapCP>), mg, dim3(64 * (4 + kMapCP)), 0, stream, ma);
  else
    hipLaunchKernelGGL((map_scan_kernel<2, kMapCP>), mg, dim3(64 * (2 + kMapCP)), 0, stream, ma);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  constexpr int kChainRows = 4;
  const SplitTables tables{tok0, ch0, a.B, a.T, nct, cps};
  hipLaunchKernelGGL(split_chain_kernel<kChainRows>, dim3((unsigned)(a.B * a.H * (128 / kChainRows))), dim3(256), 0,
                     stream, a.S0, maps, start, a.H, G, a.B * a.H, tables);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  ScanKArgs sa{};
  sa.v = vsrc;
  sa.S0 = start;
  sa.o = a.o;
  sa.S_final = end;
  sa.ws_records = records;
  sa.lay = lay;
  sa.H = a.H;
  sa.dv = a.dv;
  sa.T = a.T;
  sa.nct = nct;
  sa.seq_tok0 = tok0;
  sa.seq_chunk0 = ch0;
  sa.seq_order = nullptr;
  sa.scale = a.scale;
  sa.n_units = a.B * G * a.H;
  sa.ctl = ctl;
  sa.touch_ahead = touch;
  sa.S_last = a.S_final;  // the last segments' end states are the final states
  sa.seg_per_seq = G;
  sa.sched_id = kScheduleSplit;
  return launch_scan_phase<DK, E>(a, sa, stream);
}

template <int DK, typename E>
hipError_t run_prefill(const PrefillArgs &a, hipStream_t stream) {
  const WorkspacePlan &P = a.plan;
  const ChunkRecordLayout lay = chunk_record_layout(DK, (int)sizeof(E));
  char *records = a.ws + P.records;
  int32_t *tables = reinterpret_cast<int32_t *>(a.ws + P.tables);
  int *ctl = reinterpret_cast<int *>(a.ws);
  const bool packed = a.cu_seqlens != nullptr;
  const int nct = (a.T + kChunk - 1) / kChunk;
  const bool split = DK == 128 && sizeof(E) == 2 && !packed && P.split.G > 1 &&
                     (a.schedule == kScheduleSplit || (a.schedule == kScheduleAuto && P.split.worth));

  if (packed) {
    hipLaunchKernelGGL(varlen_index_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, P.n_seq, a.T,
                       tables + P.seq_tok0, tables + P.seq_chunk0, tables + P.chunk_t0, tables + P.chunk_len,
                       tables + P.chunk_s0, P.max_chunks, tables + P.seq_order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  if (P.max_chunks > 0) {
    PrepKArgs pa{};
    pa.q = a.q;
    pa.k = a.k;
    pa.alpha = a.alpha;
    pa.gate = a.gate;
    pa.act = a.act;
    pa.beta = a.beta;
    pa.src.T = a.T;
    pa.src.nct = nct;
    pa.src.chunk_t0 = packed ? tables + P.chunk_t0 : nullptr;
    pa.src.chunk_len = packed ? tables + P.chunk_len : nullptr;
    pa.src.chunk_s0 = packed ? tables + P.chunk_s0 : nullptr;
    pa.src.seq_chunk0 = packed ? tables + P.seq_chunk0 : nullptr;
    pa.src.n_seq = P.n_seq;
    pa.H = a.H;
    pa.scale = a.scale;
    pa.ws_records = records;
    pa.lay = lay;
    pa.ready = pa.ctl = nullptr;
    pa.ready_words = pa.n_units = 0;
    pa.conv_q = a.conv_q;
    pa.conv_k = a.conv_k;
    pa.conv_v = a.conv_v;
    pa.v = a.v;
    pa.o = a.o;
    pa.dv = a.dv;
    if (!split && overlap_supported<DK, E>(a) && overlap_chosen(a, nct)) {
      hipError_t e = hipSuccess;
      bool ran = false;
      {
        std::lock_guard<std::mutex> lock(g_overlap_mu);
        if (OverlapCtx *ov = overlap_ctx(stream)) {
          e = run_prefill_overlap<DK, E>(a, stream, pa, lay, records, *ov);
          ran = true;
        }
      }
      if (ran) return e != hipSuccess ? e : launch_out_post<E>(a, nullptr, stream);
    }
    if (P.max_chunks * a.H > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const dim3 pg((unsigned)(P.max_chunks * a.H));
    if (a.conv_q)
      launch_prep<DK, E, true, false, true>(a.gate, pg, stream, pa);
    else if (a.act & kActQK)
      launch_prep<DK, E, true>(a.gate, pg, stream, pa);
    else
      launch_prep<DK, E, false>(a.gate, pg, stream, pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.conv_q && a.conv_state && P.n_seq > 0) {
    hipLaunchKernelGGL(conv_state_kernel<E>, dim3((unsigned)(P.n_seq * a.H)), dim3(256), 0, stream,
                       reinterpret_cast<const E *>(a.q), reinterpret_cast<const E *>(a.k),
                       reinterpret_cast<const E *>(a.v), reinterpret_cast<E *>(a.conv_state), a.H, a.dk, a.dv, a.T,
                       packed ? tables + P.seq_tok0 : nullptr, P.n_seq * a.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  if constexpr (DK == 128 && sizeof(E) == 2) {
    if (split) {
      const hipError_t e = run_split<DK, E>(a, stream, records, lay);
      return e != hipSuccess ? e : launch_out_post<E>(a, nullptr, stream);
    }
  }
  if (P.n_seq > 0) {
    ScanKArgs sa{};
    sa.v = a.conv_q ? a.o : a.v;  // the prep left v's convolution in o
    sa.S0 = a.S0;
    sa.o = a.o;
    sa.S_final = a.S_final;
    sa.ws_records = records;
    sa.lay = lay;
    sa.H = a.H;
    sa.dv = a.dv;
    sa.T = a.T;
    sa.nct = nct;
    sa.seq_tok0 = packed ? tables + P.seq_tok0 : nullptr;
    sa.seq_chunk0 = packed ? tables + P.seq_chunk0 : nullptr;
    sa.seq_order = packed ? tables + P.seq_order : nullptr;
    sa.scale = a.scale;
    sa.n_units = P.n_seq * a.H;
    sa.ctl = ctl;
    // records beyond the 256 MB Infinity Cache come from HBM: touch each one
    // a step ahead (measured at d = 128 bf16 with 32 units x 256 chunks, 500
    // MB of records: 423 -> 368 us per scan; with 125 MB of records, which
    // stay in the cache, the touches cost 49 -> 52 us)
    sa.touch_ahead = DK == 128 && sizeof(E) == 2 && (size_t)P.max_chunks * a.H * lay.bytes > ((size_t)256 << 20);
    hipError_t e = launch_scan_phase<DK, E>(a, sa, stream);
    if (e != hipSuccess) return e;
  }
  return launch_out_post<E>(a, packed ? tables + P.seq_tok0 : nullptr, stream);
}

template <typename E> hipError_t run_prefill_dk(const PrefillArgs &a, hipStream_t s) {
  switch (a.dk) {
    case 16: return run_prefill<16, E>(a, s);
    case 32: return run_prefill<32, E>(a, s);
    case 64: return run_prefill<64, E>(a, s);
    case 128: return run_prefill<128, E>(a, s);
  }
  return hipErrorInvalidValue;
}

// Device scratch of kda_chunk_fwd_noalloc (prefill for callers that cannot
// allocate): one copy per device, held for the life of the process.  Host
// code never uses the array's name as an address (on the host it is a
// stand-in, not device memory): scratch_address() looks the device address
// up per device and the kernels take that pointer as their workspace.
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];  // per device, guarded by g_scratch_mu

}  // namespace

hipError_t scratch_address(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

void release_overlap() {
  std::lock_guard<std::mutex> lock(g_overlap_mu);
  auto holds = [](const OverlapCtx &c) { return c.scan || c.prep || c.fork || c.done_scan || c.done_prep; };
  bool any = false;
  for (const OverlapCtx &c : g_overlap) any = any || holds(c);
  if (!any) {  // nothing was created: no runtime call at all
    for (OverlapCtx &c : g_overlap) c = OverlapCtx{};
    return;
  }
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (int dev = 0; dev < 64; ++dev) {
    OverlapCtx &c = g_overlap[dev];
    if (holds(c) && hipSetDevice(dev) == hipSuccess) {
      // work still queued on the streams finishes before they go
      if (c.scan) (void)hipStreamSynchronize(c.scan);
      if (c.prep) (void)hipStreamSynchronize(c.prep);
      destroy_ctx(c);
    }
    c = OverlapCtx{};
  }
  if (have_cur) (void)hipSetDevice(cur);
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  return a.bf16 ? run_prefill_dk<bf16>(a, stream) : run_prefill_dk<float>(a, stream);
}

hipError_t launch_out_norm_gate(void *o, const void *gate, const float *w, float eps, int H, long long n_tok, int dv,
                                bool is_bf16, hipStream_t stream) {
  return is_bf16 ? launch_norm_gate_rows<bf16>(o, gate, w, eps, H, n_tok, dv, nullptr, 0, stream)
                 : launch_norm_gate_rows<float>(o, gate, w, eps, H, n_tok, dv, nullptr, 0, stream);
}

}  // namespace kda
