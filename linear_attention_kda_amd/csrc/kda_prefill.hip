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

#include <cstdlib>
#include <type_traits>

namespace kda {
namespace {

// ============================================================ index kernel
// Packed batch -> monotone clamped sequence offsets, chunk counts and the
// chunk list.  Offsets are clamped to [0, T] and made non-decreasing, so every
// token index used later stays inside the buffers even for malformed input.
__global__ __launch_bounds__(1024) void varlen_index_kernel(
    const int32_t *__restrict__ cu, int N, int T, int32_t *seq_tok0,
    int32_t *seq_chunk0, int32_t *chunk_t0, int32_t *chunk_len,
    long long max_chunks) {
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
        }
      }
    }
    tok_carry = next_tok_carry;
    chunk_carry = next_chunk_carry;
    __syncthreads();
  }
  if (tid == 0) seq_chunk0[N] = chunk_carry;
}

struct ChunkSource {
  // dense batch: sequence n starts at token n*T, nct chunks per sequence
  int T, nct;
  // packed batch (device tables; null for dense)
  const int32_t *chunk_t0, *chunk_len, *seq_chunk0;
  int n_seq;
};

__device__ __forceinline__ bool chunk_span(const ChunkSource &cs, long long c,
                                           long long &t0, int &L) {
  if (cs.chunk_t0) {
    if (c >= cs.seq_chunk0[cs.n_seq]) return false;
    t0 = cs.chunk_t0[c];
    L = cs.chunk_len[c];
  } else {
    const long long n = c / cs.nct, ci = c % cs.nct;
    t0 = n * cs.T + ci * kChunk;
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

// Copy a 64 x 64 tile from padded LDS rows (stride ld) to fragment order.
template <typename E>
__device__ __forceinline__ void lds_to_global_frag64(E *dst, const E *src, int ld) {
  for (int idx = threadIdx.x; idx < 64 * 64; idx += kThreads) {
    const int i = idx >> 6, c = idx & 63;
    dst[frag_index<E, 64>(i, c)] = src[i * ld + c];
  }
}

// ======================================================= kernel 1: chunk prep
struct PrepKArgs {
  const void *q, *k;
  const float *alpha, *beta;
  ChunkSource src;
  int H;
  float scale;
  char *ws_records;
  ChunkRecordLayout lay;
};

template <int DK, typename E> struct PrepSmem {
  static constexpr int PAD = sizeof(E) == 2 ? 8 : 4;
  static constexpr int LD = DK + PAD;    // rows of the 64 x d_k operand tiles
  static constexpr int LDT = 64 + PAD;   // rows of 64-wide E tiles
  static constexpr int LDR = 68;         // rows of fp32 64x64 tiles
  static constexpr size_t a_bytes = (size_t)4 * 64 * LD * sizeof(E);
  static constexpr size_t b_bytes = (size_t)2 * 64 * LDR * sizeof(float) + (size_t)64 * LDT * sizeof(E);
  static constexpr size_t bytes = a_bytes > b_bytes ? a_bytes : b_bytes;
};

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

// One 16x16 tile of A^kk or A^qk over d_k on the matrix cores, with the B rows
// optionally scaled per key channel by f (fp32, LDS) on the way in.
template <typename M, int K, typename E>
__device__ __forceinline__ f32x4 mma_rows_scaled(const E *a_row, const E *bt_row, const float *f, f32x4 acc) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += M::KS) {
    typename M::frag b = M::load(bt_row + k0 + g * M::KPL);
    if (f) {
#pragma unroll
      for (int e = 0; e < M::KPL; ++e) {
        if constexpr (M::KPL == 1) b = b * f[k0 + g];
        else b[e] = (E)((float)b[e] * f[k0 + g * M::KPL + e]);
      }
    }
    acc = M::mma(M::load(a_row + k0 + g * M::KPL), b, acc);
  }
  return acc;
}

// tile t in 0..9 -> (I, J) of the lower block triangle, row-major
__device__ __forceinline__ void tile_ij(int t, int &I, int &J) {
  I = t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0));
  J = t - I * (I + 1) / 2;
}

// Chunk prep.  The chunk is cut into four blocks of 16 tokens.  Per key
// channel: a_i = in-block inclusive prefix product of the gates, s_j = in-block
// exclusive suffix product, tau_b = whole-block product.  Then for j <= i
//   D_{j+1:i} = a_i / a_j                                    (same block)
//   D_{j+1:i} = s_j * prod_{J<b<I} tau_b * a_i               (block J < block I)
// The second form has no division and no factor above 1, so off-diagonal
// blocks are safe for any gates.  The first form is used on a diagonal block
// while its tau >= 2^-100 on every channel; otherwise that block is formed
// exactly with running products.
template <int DK, typename E>
__global__ __launch_bounds__(kThreads) void chunk_prep_kernel(PrepKArgs a) {
  typedef PrepSmem<DK, E> SM;
  constexpr int LD = SM::LD, LDT = SM::LDT, LDR = SM::LDR;
  typedef typename MmaFor<E, DK>::type M;
  constexpr int NTASK = 4 * DK;                               // (channel, block) pairs
  constexpr int TPT = (NTASK + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) char smem[SM::bytes];
  __shared__ __attribute__((aligned(16))) float sTau[4 * DK];  // tau_b per channel
  __shared__ __attribute__((aligned(16))) float sF[3 * DK];    // tau_1, tau_2, tau_1*tau_2
  __shared__ float sBeta[kChunk];
  __shared__ int sFlag[4];

  E *sKr = reinterpret_cast<E *>(smem);   // k_i a_i           (left operand)
  E *sQr = sKr + 64 * LD;                 // q_i a_i           (left operand)
  E *sKl = sQr + 64 * LD;                 // k_j s_j           (right, off-diagonal)
  E *sKd = sKl + 64 * LD;                 // k_j / a_j         (right, diagonal)
  float *sR = reinterpret_cast<float *>(smem);
  float *sT = sR + 64 * LDR;
  E *sOut = reinterpret_cast<E *>(sT + 64 * LDR);

  const int h = blockIdx.y;
  const long long c = blockIdx.x;
  long long t0;
  int L;
  if (!chunk_span(a.src, c, t0, L)) return;

  char *rec = a.ws_records + ((size_t)c * a.H + h) * a.lay.bytes;
  const int tid = threadIdx.x, w = wave_id(), l = lane_id();
  const E *q = reinterpret_cast<const E *>(a.q);
  const E *k = reinterpret_cast<const E *>(a.k);
  const size_t hs = (size_t)a.H * DK;  // token stride of q, k, alpha
  const size_t base = (size_t)t0 * hs + (size_t)h * DK;
  E *gKh = reinterpret_cast<E *>(rec + a.lay.kh);
  E *gQh = reinterpret_cast<E *>(rec + a.lay.qh);
  E *gKtT = reinterpret_cast<E *>(rec + a.lay.ktt);

  if (tid < kChunk) sBeta[tid] = tid < L ? a.beta[(size_t)(t0 + tid) * a.H + h] : 0.f;
  if (tid < 4) sFlag[tid] = 0;

  // ---- per (channel, block): load, in-block prefix / suffix products.
  // Padded tokens (index >= L) have q = k = 0 and alpha = 1.
  float kv[TPT][16], qv[TPT][16], pa[TPT][16], ps[TPT][16];
#pragma unroll
  for (int m = 0; m < TPT; ++m) {
    const int p = tid + kThreads * m;
    if (p < NTASK) {
      const int ch = p % DK, b = p / DK;
      float av[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // branch-free: load a valid token, then substitute the padding values
        const int tok = 16 * b + i;
        const bool live = tok < L;
        const size_t off = base + (size_t)min(tok, L - 1) * hs + ch;
        const float al = a.alpha[off], kx = to_f(k[off]), qx = to_f(q[off]);
        av[i] = live ? al : 1.f;
        kv[m][i] = live ? kx : 0.f;
        qv[m][i] = live ? qx : 0.f;
      }
      float run = 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        run *= av[i];
        pa[m][i] = run;
      }
      run = 1.f;
#pragma unroll
      for (int j = 15; j >= 0; --j) {
        ps[m][j] = run;
        run *= av[j];
      }
    }
  }
  __syncthreads();  // sFlag initialised
#pragma unroll
  for (int m = 0; m < TPT; ++m) {
    const int p = tid + kThreads * m;
    if (p < NTASK) {
      const int ch = p % DK, b = p / DK;
      const float tau = pa[m][15];
      sTau[b * DK + ch] = tau;
      if (!(tau >= 0x1p-100f)) sFlag[b] = 1;
    }
  }
  __syncthreads();

  // ---- operands: LDS tiles for A^kk / A^qk, record tiles for the scan
#pragma unroll
  for (int m = 0; m < TPT; ++m) {
    const int p = tid + kThreads * m;
    if (p < NTASK) {
      const int ch = p % DK, b = p / DK;
      const float t0_ = sTau[ch], t1_ = sTau[DK + ch], t2_ = sTau[2 * DK + ch], t3_ = sTau[3 * DK + ch];
      // D_{0:16b-1} (blocks before b) and D_{16b+16:63} (blocks after b)
      const float fb = b == 0 ? 1.f : (b == 1 ? t0_ : (b == 2 ? t0_ * t1_ : t0_ * t1_ * t2_));
      const float gb = b == 3 ? 1.f : (b == 2 ? t3_ : (b == 1 ? t2_ * t3_ : t1_ * t2_ * t3_));
      if (b == 0) {
        reinterpret_cast<float *>(rec + a.lay.p63)[ch] = t0_ * t1_ * t2_ * t3_;
        sF[ch] = t1_;
        sF[DK + ch] = t2_;
        sF[2 * DK + ch] = t1_ * t2_;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 16 * b + i;
        const float kr = kv[m][i] * pa[m][i], qr = qv[m][i] * pa[m][i];
        sKr[row * LD + ch] = from_f<E>(kr);
        sQr[row * LD + ch] = from_f<E>(qr);
        sKl[row * LD + ch] = from_f<E>(kv[m][i] * ps[m][i]);
        sKd[row * LD + ch] = from_f<E>(kv[m][i] * __builtin_amdgcn_rcpf(pa[m][i]));
        gKh[frag_index<E, DK>(row, ch)] = from_f<E>(kr * fb);                  // k_i D_{0:i}
        gQh[frag_index<E, DK>(row, ch)] = from_f<E>(qr * fb * a.scale);        // s q_i D_{0:i}
        gKtT[frag_index<E, 64>(ch, row)] = from_f<E>(kv[m][i] * ps[m][i] * gb);  // k_j D_{j+1:63}
      }
    }
  }
  __syncthreads();

  // ---- A^kk (tiles 0..9) and A^qk (tiles 10..19), lower block triangle
  f32x4 acc[5];
#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const int t = w + 4 * s, kind = t / 10;
    int I, J;
    tile_ij(t % 10, I, J);
    const E *arow = (kind == 0 ? sKr : sQr) + (16 * I + (l & 15)) * LD;
    const E *brow = (I == J ? sKd : sKl) + (16 * J + (l & 15)) * LD;
    const float *f = I - J == 2 ? sF + (J == 0 ? 0 : DK) : (I - J == 3 ? sF + 2 * DK : nullptr);
    acc[s] = mma_rows_scaled<M, DK>(arow, brow, f, zero4());
  }
  __syncthreads();  // the operand area is reused from here on

#pragma unroll
  for (int s = 0; s < 5; ++s) {
    const int t = w + 4 * s, kind = t / 10;
    int I, J;
    tile_ij(t % 10, I, J);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * (l >> 4) + r, j = 16 * J + (l & 15);
      if (kind == 0)
        sR[i * LDR + j] = j < i ? sBeta[i] * acc[s][r] : 0.f;
      else
        sOut[i * LDT + j] = from_f<E>(j <= i ? a.scale * acc[s][r] : 0.f);
    }
  }
  // zero the blocks of A above the diagonal
  for (int idx = tid; idx < 6 * 256; idx += kThreads) {
    const int u = idx >> 8, e = idx & 255;
    const int I = u < 3 ? 0 : (u < 5 ? 1 : 2);
    const int J = u < 3 ? u + 1 : (u < 5 ? u - 1 : 3);
    sOut[(16 * I + (e >> 4)) * LDT + 16 * J + (e & 15)] = from_f<E>(0.f);
  }
  __syncthreads();

  // ---- exact diagonal blocks where the in-block decay left fp32's range:
  // thread (j, channel group) runs D_{j+1:i} as a product over i.
  for (int b = 0; b < 4; ++b) {
    if (!sFlag[b]) continue;  // uniform: read after a barrier
    constexpr int CPG = DK / 16;
    const int j = tid >> 4, cg = tid & 15, s0 = 16 * b;
    float racc[16], aacc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) racc[i] = aacc[i] = 0.f;
    for (int cc = 0; cc < CPG; ++cc) {
      const int ch = cg * CPG + cc;
      const float kj = s0 + j < L ? to_f(k[base + (size_t)(s0 + j) * hs + ch]) : 0.f;
      float rho = 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i >= j && s0 + i < L) {
          const size_t off = base + (size_t)(s0 + i) * hs + ch;
          if (i > j) rho *= a.alpha[off];
          const float wgt = kj * rho;
          if (i > j) racc[i] += to_f(k[off]) * wgt;
          aacc[i] += to_f(q[off]) * wgt;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
        racc[i] += __shfl_xor(racc[i], m);
        aacc[i] += __shfl_xor(aacc[i], m);
      }
    }
    if (cg == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sR[(s0 + i) * LDR + s0 + j] = i > j ? sBeta[s0 + i] * racc[i] : 0.f;
        sOut[(s0 + i) * LDT + s0 + j] = from_f<E>(i >= j ? a.scale * aacc[i] : 0.f);
      }
    }
    __syncthreads();
  }
  lds_to_global_frag64(reinterpret_cast<E *>(rec + a.lay.aqk), sOut, LDT);

  // ---- T = (I + R)^{-1}: diagonal 16x16 blocks by forward substitution.
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
  }
  __syncthreads();
  if (w < 3) inverse_offdiag_block<LDR>(w + 1, w, sR, sT);  // (1,0) (2,1) (3,2)
  __syncthreads();
  if (w < 2) inverse_offdiag_block<LDR>(w + 2, w, sR, sT);  // (2,0) (3,1)
  __syncthreads();
  if (w == 0) inverse_offdiag_block<LDR>(3, 0, sR, sT);     // (3,0)
  __syncthreads();

  // ---- Tb = T Diag(beta), zero above the diagonal
  for (int idx = tid; idx < 64 * 64; idx += kThreads) {
    const int i = idx >> 6, j = idx & 63;
    sOut[i * LDT + j] = from_f<E>(j <= i ? sT[i * LDR + j] * sBeta[j] : 0.f);
  }
  __syncthreads();
  lds_to_global_frag64(reinterpret_cast<E *>(rec + a.lay.tb), sOut, LDT);
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
  float scale;
  int n_units;                           // sequences * heads
  int wg_per_unit;                       // workgroups per unit (value tiles / waves per WG)
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
    for (int u = 0; u < (KU + F::W - 1) / F::W; ++u) {
      if constexpr (F::wide)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.x[u], f[u], acc, 0, 0, 0);
      else
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.x[u], f[u], acc, 0, 0, 0);
    }
    return acc;
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
    for (int u = 0; u < (KU + 15) / 16; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x[u][s], f[u][s], acc, 0, 0, 0);
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

// Compile-time copy of ChunkRecordLayout for the scan's LDS image of a record.
template <int DK, typename E> struct RecordShape {
  static constexpr int es = sizeof(E);
  static constexpr int kh = 0, qh = 64 * DK * es, ktt = 128 * DK * es, tb = 192 * DK * es;
  static constexpr int aqk = tb + 4096 * es, p63 = aqk + 4096 * es;
  static constexpr int bytes = (p63 + DK * 4 + 1023) / 1024 * 1024;
};

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
template <int DK, typename E, int NT, int CW>
__global__ __launch_bounds__(64 * (CW + 1)) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunk_scan_kernel(ScanKArgs a) {
  typedef RecordShape<DK, E> RS;
  constexpr int CT = DK / 16;
  constexpr int VC = 16 * NT;                   // value columns per compute wave
  typedef FragShape<E, DK> FK;   // products over d_k
  typedef FragShape<E, 64> FT;   // products over the 64 tokens
  constexpr int TILE_K = FK::NU * 64 * FK::KS;   // elements per 16-row tile, K = d_k
  constexpr int TILE_T = FT::NU * 64 * FT::KS;   // elements per 16-row tile, K = 64
  constexpr int VSL = 64 * VC;                   // value-slice elements per compute wave
  constexpr int STAGE = RS::bytes + CW * VSL * (int)sizeof(E);
  constexpr int NBUF = 2 * STAGE <= 160 * 1024 ? 2 : 1;   // double buffer if it fits
  static_assert(STAGE <= 160 * 1024 - 1024, "one stage must fit in LDS");
  __shared__ __attribute__((aligned(1024))) char rec0[RS::bytes];
  __shared__ __attribute__((aligned(1024))) char rec1[NBUF == 2 ? RS::bytes : 1024];
  __shared__ __attribute__((aligned(16))) E vsl0[CW * VSL];
  __shared__ __attribute__((aligned(16))) E vsl1[NBUF == 2 ? CW * VSL : 8];

  const int w = wave_id(), l = lane_id(), col = l & 15, g = l >> 4;
  const int bid = blockIdx.x, xcd = bid & 7, slot = bid >> 3;
  const int u = (slot / a.wg_per_unit) * 8 + xcd;
  if (u >= a.n_units) return;
  const int n = u / a.H, h = u % a.H;
  const int vwg = (slot % a.wg_per_unit) * (CW * VC);  // first value column of the workgroup
  const int H = a.H, DV = a.dv;
  const bool copier = w == CW;

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
  // Value slices land as [compute wave][16-byte column group][token][elements];
  // rows past the end of the sequence repeat its last token (they never reach
  // a valid output: their Tb rows and columns are zero).
  constexpr int VE = 16 / (int)sizeof(E);        // elements per 16-byte group
  constexpr int VG = VC / VE;                    // 16-byte groups per value row
  auto copy_chunk = [&](int ci, char *rec, E *vsl) {
    const char *src = a.ws_records + ((size_t)(chunk0 + ci) * H + h) * RS::bytes + l * 16;
    const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) char *)rec;
    for (int q = 0; q < RS::bytes / 1024; ++q) lds_dma16(src + q * 1024, lds + q * 1024);
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const E *vsrc = V + (size_t)(t0 + min(l, L - 1)) * tok_stride + (size_t)h * DV + vwg;
    const uint32_t vl = (uint32_t)(size_t)(__attribute__((address_space(3))) E *)vsl;
#pragma unroll
    for (int cw = 0; cw < CW; ++cw)
#pragma unroll
      for (int q = 0; q < VG; ++q)
        lds_dma16(vsrc + cw * VC + q * VE, vl + (uint32_t)((cw * VSL + q * 64 * VE) * sizeof(E)));
  };
  if (copier) {
    if (NBUF == 2) {
      if (nchunks > 0) copy_chunk(0, rec0, vsl0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // chunk 0 ready
      for (int ci = 0; ci < nchunks; ++ci) {
        // buffer (ci+1)%2 held chunk ci-1, which every compute wave finished
        // before the barrier that ended the previous step
        if (ci + 1 < nchunks) {
          if (ci & 1) copy_chunk(ci + 1, rec0, vsl0);
          else copy_chunk(ci + 1, rec1, vsl1);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();  // chunk ci done by the compute waves, chunk ci+1 ready
      }
    } else {
      for (int ci = 0; ci < nchunks; ++ci) {
        __syncthreads();  // buffer free
        copy_chunk(ci, rec0, vsl0);
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

  // One chunk.  LDS operand reads are issued in the order the products use
  // them; the scheduler is held to a pattern that keeps reads ahead of the
  // matrix cores while bounding the registers the fragments take.
  auto compute = [&](const char *recb, const E *vs, f32x4 (*ov)[NT]) {
    typedef BOps<E, DK> BK;
    typedef BOps<E, 64> BT;
    const E *Kh = reinterpret_cast<const E *>(recb + RS::kh);
    const E *Qh = reinterpret_cast<const E *>(recb + RS::qh);
    const E *KtT = reinterpret_cast<const E *>(recb + RS::ktt);
    const E *Tb = reinterpret_cast<const E *>(recb + RS::tb);
    const E *Aq = reinterpret_cast<const E *>(recb + RS::aqk);
    const float *P63 = reinterpret_cast<const float *>(recb + RS::p63);
    vs += w * VSL;

    // X_top = Kbnd S^T, X_bot = s Qbnd S^T
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
    for (int I = 0; I < 4; ++I) {
      const typename BK::template A<DK> fk = BK::template load<DK>(Kh + I * TILE_K);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) xt[I][nt] = sb[nt].mma(fk, zero4());
      const typename BK::template A<DK> fq = BK::template load<DK>(Qh + I * TILE_K);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) xb[I][nt] = sb[nt].mma(fq, zero4());
    }
    // Ebar = V - X_top ; E = Tb Ebar (row block I needs columns < 16(I+1))
    BT ebo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 eb[4];
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = 16 * nt + col;
          eb[I][r] = to_f(vs[((c / VE) * 64 + 16 * I + 4 * g + r) * VE + c % VE]) - xt[I][nt][r];
        }
      ebo[nt].build(eb);
    }
    f32x4 e[4][NT];
    {
      const typename BT::template A<16> f0 = BT::template load<16>(Tb + 0 * TILE_T);
      const typename BT::template A<32> f1 = BT::template load<32>(Tb + 1 * TILE_T);
      const typename BT::template A<48> f2 = BT::template load<48>(Tb + 2 * TILE_T);
      const typename BT::template A<64> f3 = BT::template load<64>(Tb + 3 * TILE_T);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        e[0][nt] = ebo[nt].mma(f0, zero4());
        e[1][nt] = ebo[nt].mma(f1, zero4());
        e[2][nt] = ebo[nt].mma(f2, zero4());
        e[3][nt] = ebo[nt].mma(f3, zero4());
      }
    }
    // O = s Qbnd S^T + A E
    BT eo[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 et[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) et[I] = e[I][nt];
      eo[nt].build(et);
    }
    {
      const typename BT::template A<16> f0 = BT::template load<16>(Aq + 0 * TILE_T);
      const typename BT::template A<32> f1 = BT::template load<32>(Aq + 1 * TILE_T);
      const typename BT::template A<48> f2 = BT::template load<48>(Aq + 2 * TILE_T);
      const typename BT::template A<64> f3 = BT::template load<64>(Aq + 3 * TILE_T);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        ov[0][nt] = eo[nt].mma(f0, xb[0][nt]);
        ov[1][nt] = eo[nt].mma(f1, xb[1][nt]);
        ov[2][nt] = eo[nt].mma(f2, xb[2][nt]);
        ov[3][nt] = eo[nt].mma(f3, xb[3][nt]);
      }
    }
    // S^T = D_{0:63} S^T + Kend^T E
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const f32x4 p = *reinterpret_cast<const f32x4 *>(P63 + 16 * ct + 4 * g);
      const typename BT::template A<64> fkt = BT::template load<64>(KtT + ct * TILE_T);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) st[ct][nt][r] *= p[r];
        st[ct][nt] = eo[nt].mma(fkt, st[ct][nt]);
      }
    }
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
          if constexpr (sizeof(E) == 2)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f<E>(x)), rs,
                                                  o_lane + row_off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), rs, o_lane + row_off, 0, 0);
        }
    }
  };

  f32x4 ov[4][NT];
  if (NBUF == 2) {
    __syncthreads();  // chunk 0 ready
    for (int ci = 0; ci < nchunks; ci += 2) {
      if (ci > 0) store_o(ci - 1, ov);
      compute(rec0, vsl0, ov);
      __syncthreads();
      if (ci + 1 >= nchunks) break;
      store_o(ci, ov);
      compute(rec1, vsl1, ov);
      __syncthreads();
    }
  } else {
    for (int ci = 0; ci < nchunks; ++ci) {
      __syncthreads();  // buffer free
      if (ci > 0) store_o(ci - 1, ov);
      __syncthreads();  // buffer ready
      compute(rec0, vsl0, ov);
    }
  }
  if (nchunks > 0) store_o(nchunks - 1, ov);

#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      *reinterpret_cast<f32x4 *>(a.S_final + sbase + (size_t)16 * nt * DK + 16 * ct + 4 * g) = st[ct][nt];
}

// LDS held by one stage (record + value slices) of a scan configuration.
template <int DK, typename E> constexpr bool scan_stage_fits(int nt, int cw) {
  return RecordShape<DK, E>::bytes + cw * 64 * 16 * nt * (int)sizeof(E) <= 160 * 1024 - 1024;
}

template <int DK, typename E, int NT>
void launch_scan(int cw, dim3 grid, dim3 block, hipStream_t stream, const ScanKArgs &sa) {
  if constexpr (scan_stage_fits<DK, E>(NT, 4))
    if (cw == 4) {
      hipLaunchKernelGGL((chunk_scan_kernel<DK, E, NT, 4>), grid, block, 0, stream, sa);
      return;
    }
  if constexpr (scan_stage_fits<DK, E>(NT, 2))
    if (cw == 2) {
      hipLaunchKernelGGL((chunk_scan_kernel<DK, E, NT, 2>), grid, block, 0, stream, sa);
      return;
    }
  hipLaunchKernelGGL((chunk_scan_kernel<DK, E, NT, 1>), grid, block, 0, stream, sa);
}

// ================================================================ dispatch
template <int DK, typename E>
hipError_t run_prefill(const PrefillArgs &a, hipStream_t stream) {
  const WorkspacePlan &P = a.plan;
  const ChunkRecordLayout lay = chunk_record_layout(DK, (int)sizeof(E));
  char *records = a.ws + P.tables_bytes;
  int32_t *tables = reinterpret_cast<int32_t *>(a.ws);
  const bool packed = a.cu_seqlens != nullptr;
  const int nct = (a.T + kChunk - 1) / kChunk;

  if (packed) {
    hipLaunchKernelGGL(varlen_index_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, P.n_seq, a.T,
                       tables + P.seq_tok0, tables + P.seq_chunk0, tables + P.chunk_t0, tables + P.chunk_len,
                       P.max_chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  if (P.max_chunks > 0) {
    PrepKArgs pa;
    pa.q = a.q;
    pa.k = a.k;
    pa.alpha = a.alpha;
    pa.beta = a.beta;
    pa.src.T = a.T;
    pa.src.nct = nct;
    pa.src.chunk_t0 = packed ? tables + P.chunk_t0 : nullptr;
    pa.src.chunk_len = packed ? tables + P.chunk_len : nullptr;
    pa.src.seq_chunk0 = packed ? tables + P.seq_chunk0 : nullptr;
    pa.src.n_seq = P.n_seq;
    pa.H = a.H;
    pa.scale = a.scale;
    pa.ws_records = records;
    pa.lay = lay;
    hipLaunchKernelGGL((chunk_prep_kernel<DK, E>), dim3((unsigned)P.max_chunks, a.H), dim3(kThreads), 0, stream,
                       pa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  if (P.n_seq > 0) {
    ScanKArgs sa;
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
    sa.seq_tok0 = packed ? tables + P.seq_tok0 : nullptr;
    sa.seq_chunk0 = packed ? tables + P.seq_chunk0 : nullptr;
    sa.scale = a.scale;
    sa.n_units = P.n_seq * a.H;
    // compute waves per workgroup (CW) and 16-column tiles per wave (NT).
    // Two tiles per wave halve the LDS reads per column but double each
    // wave's serial chain of products; one tile and two compute waves per
    // workgroup measured fastest at d_v = 128.
    int nt = 1, cw = a.dv >= 32 ? 2 : 1;
    if (const char *env = std::getenv("KDA_SCAN_NT")) {
      const int x = std::atoi(env);
      if ((x == 1 || x == 2) && 16 * x <= a.dv) nt = x;
    }
    if (const char *env = std::getenv("KDA_SCAN_CW")) {
      const int x = std::atoi(env);
      if (x == 1 || x == 2 || x == 4) cw = x;
    }
    while (cw > 1 && (16 * nt * cw > a.dv || !scan_stage_fits<DK, E>(nt, cw))) cw /= 2;
    sa.wg_per_unit = a.dv / (16 * nt * cw);
    const long long slots = ((long long)sa.n_units + 7) / 8 * 8 * sa.wg_per_unit;
    const dim3 grid((unsigned)slots);
    const dim3 block(64 * (cw + 1));
    if (nt == 2)
      launch_scan<DK, E, 2>(cw, grid, block, stream, sa);
    else
      launch_scan<DK, E, 1>(cw, grid, block, stream, sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
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

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream) {
  return a.bf16 ? run_prefill_dk<bf16>(a, stream) : run_prefill_dk<float>(a, stream);
}

}  // namespace kda
