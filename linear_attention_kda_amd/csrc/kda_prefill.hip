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
//   kernel 2 (scan, one workgroup per (sequence, head, d_v tile)): walks the
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

// Copy `rows` rows of `rowlen` elements from padded LDS rows (stride ld) to a
// dense global array, 16 bytes per thread per step.
template <typename E>
__device__ __forceinline__ void lds_to_global(char *dst, const E *src, int rows, int rowlen, int ld) {
  const int vpr = rowlen * (int)sizeof(E) / 16;
  for (int idx = threadIdx.x; idx < rows * vpr; idx += kThreads) {
    const int r = idx / vpr, cv = idx % vpr;
    *reinterpret_cast<uint4 *>(dst + ((size_t)r * rowlen * sizeof(E)) + cv * 16) =
        *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(src + r * ld) + cv * 16);
  }
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
        const int tok = 16 * b + i;
        av[i] = 1.f;
        kv[m][i] = qv[m][i] = 0.f;
        if (tok < L) {
          const size_t off = base + (size_t)tok * hs + ch;
          av[i] = a.alpha[off];
          kv[m][i] = to_f(k[off]);
          qv[m][i] = to_f(q[off]);
        }
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
      E kt[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 16 * b + i;
        const float kr = kv[m][i] * pa[m][i], qr = qv[m][i] * pa[m][i];
        sKr[row * LD + ch] = from_f<E>(kr);
        sQr[row * LD + ch] = from_f<E>(qr);
        sKl[row * LD + ch] = from_f<E>(kv[m][i] * ps[m][i]);
        sKd[row * LD + ch] = from_f<E>(kv[m][i] * __builtin_amdgcn_rcpf(pa[m][i]));
        gKh[(size_t)row * DK + ch] = from_f<E>(kr * fb);   // k_i D_{0:i}
        gQh[(size_t)row * DK + ch] = from_f<E>(qr * fb);   // q_i D_{0:i}
        kt[i] = from_f<E>(kv[m][i] * ps[m][i] * gb);       // k_j D_{j+1:63}
      }
      // row ch of Kend^T, columns 16b..16b+15: contiguous
      uint4 *dst = reinterpret_cast<uint4 *>(gKtT + (size_t)ch * 64 + 16 * b);
      const uint4 *srcv = reinterpret_cast<const uint4 *>(kt);
#pragma unroll
      for (int v4 = 0; v4 < (int)(16 * sizeof(E) / 16); ++v4) dst[v4] = srcv[v4];
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
  lds_to_global(rec + a.lay.aqk, sOut, 64, 64, LDT);

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
  lds_to_global(rec + a.lay.tb, sOut, 64, 64, LDT);
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
};

template <int DK, int BV, typename E>
__global__ __launch_bounds__(kThreads) void chunk_scan_kernel(ScanKArgs a) {
  typedef typename MmaFor<E, DK>::type MK;  // products over d_k
  typedef Mma<E, 32> MC;                    // products over the 64 tokens
  constexpr int NB = BV / 16;               // value-column tiles
  constexpr int CT = DK / 16;               // key-channel tiles of the state
  constexpr int CTW = (CT + 3) / 4;         // state tiles per wave
  constexpr int PAD = sizeof(E) == 2 ? 8 : 4;
  constexpr int LDS_ = DK + PAD, LDE = 64 + PAD;
  __shared__ __attribute__((aligned(16))) E sS[BV * LDS_];   // S (bf16/fp32 copy), [v][c]
  __shared__ __attribute__((aligned(16))) E sEb[BV * LDE];   // Ebar^T, [v][i]
  __shared__ __attribute__((aligned(16))) E sE[BV * LDE];    // E^T, [v][i]

  const int vt = blockIdx.x, h = blockIdx.y, n = blockIdx.z;
  const int w = wave_id(), l = lane_id(), col = l & 15, g = l >> 4;
  const int v0 = vt * BV;
  const int H = a.H, DV = a.dv;

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

  // ---- state S^T tiles owned by this wave: channel tile ct = w*CTW + u
  const size_t sbase = ((size_t)n * H + h) * DV * DK;
  f32x4 st[CTW][NB];
#pragma unroll
  for (int u = 0; u < CTW; ++u) {
    const int ct = w * CTW + u;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      st[u][nb] = zero4();
      if (ct < CT) {
        const int vv = 16 * nb + col, c4 = 16 * ct + 4 * g;
        if (a.S0) st[u][nb] = *reinterpret_cast<const f32x4 *>(a.S0 + sbase + (size_t)(v0 + vv) * DK + c4);
#pragma unroll
        for (int r = 0; r < 4; ++r) sS[vv * LDS_ + c4 + r] = from_f<E>(st[u][nb][r]);
      }
    }
  }
  __syncthreads();

  const E *V = reinterpret_cast<const E *>(a.v);
  E *O = reinterpret_cast<E *>(a.o);
  const size_t tok_stride = (size_t)H * DV;

  for (int ci = 0; ci < nchunks; ++ci) {
    const char *rec = a.ws_records + ((size_t)(chunk0 + ci) * H + h) * a.lay.bytes;
    const long long t0 = tstart + (long long)kChunk * ci;
    const int L = (int)min((long long)kChunk, ntok - (long long)kChunk * ci);
    const E *Kh = reinterpret_cast<const E *>(rec + a.lay.kh);
    const E *Qh = reinterpret_cast<const E *>(rec + a.lay.qh);
    const E *KtT = reinterpret_cast<const E *>(rec + a.lay.ktt);
    const E *Tb = reinterpret_cast<const E *>(rec + a.lay.tb);
    const E *Aqk = reinterpret_cast<const E *>(rec + a.lay.aqk);
    const float *P63 = reinterpret_cast<const float *>(rec + a.lay.p63);

    // ---- X = [Kbnd; Qbnd] S^T: wave w takes rows 32w..32w+31 of the stack
    const E *Xsrc = w < 2 ? Kh + (size_t)(32 * w) * DK : Qh + (size_t)(32 * (w - 2)) * DK;
    f32x4 x[2][NB];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        x[rt][nb] = mma_rows<MK, DK>(Xsrc + (size_t)(16 * rt + col) * DK, sS + (16 * nb + col) * LDS_, zero4());

    // ---- Ebar = V - Kbnd S^T  (waves 0, 1), stored transposed
    if (w < 2) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int vv = 16 * nb + col, i0 = 32 * w + 16 * rt + 4 * g;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = i0 + r;
            const float vval = i < L ? to_f(V[(size_t)(t0 + i) * tok_stride + (size_t)h * DV + v0 + vv]) : 0.f;
            sEb[vv * LDE + i] = from_f<E>(vval - x[rt][nb][r]);
          }
        }
    }
    __syncthreads();

    // ---- E = Tb Ebar: wave w takes rows 16w..16w+15
    {
      f32x4 e[NB];
      const E *trow = Tb + (size_t)(16 * w + col) * 64;
      const int kend = 16 * (w + 1);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        e[nb] = zero4();
        const E *brow = sEb + (16 * nb + col) * LDE;
        for (int k0 = 0; k0 < kend; k0 += MC::KS)
          e[nb] = MC::mma(MC::load(trow + k0 + g * MC::KPL), MC::load(brow + k0 + g * MC::KPL), e[nb]);
#pragma unroll
        for (int r = 0; r < 4; ++r) sE[(16 * nb + col) * LDE + 16 * w + 4 * g + r] = from_f<E>(e[nb][r]);
      }
    }
    __syncthreads();

    // ---- O = s Qbnd S^T + A E  (waves 2, 3)
    if (w >= 2) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const int rb = 32 * (w - 2) + 16 * rt;
        const E *arow = Aqk + (size_t)(rb + col) * 64;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          f32x4 ov;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = a.scale * x[rt][nb][r];
          const E *brow = sE + (16 * nb + col) * LDE;
          for (int k0 = 0; k0 < rb + 16; k0 += MC::KS)
            ov = MC::mma(MC::load(arow + k0 + g * MC::KPL), MC::load(brow + k0 + g * MC::KPL), ov);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = rb + 4 * g + r;
            if (i < L) O[(size_t)(t0 + i) * tok_stride + (size_t)h * DV + v0 + 16 * nb + col] = from_f<E>(ov[r]);
          }
        }
      }
    }

    // ---- S^T = D_{0:63} S^T + Kend^T E
#pragma unroll
    for (int u = 0; u < CTW; ++u) {
      const int ct = w * CTW + u;
      if (ct < CT) {
        const f32x4 p = *reinterpret_cast<const f32x4 *>(P63 + 16 * ct + 4 * g);
        const E *arow = KtT + (size_t)(16 * ct + col) * 64;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) st[u][nb][r] *= p[r];
          st[u][nb] = mma_rows<MC, 64>(arow, sE + (16 * nb + col) * LDE, st[u][nb]);
          const int vv = 16 * nb + col, c4 = 16 * ct + 4 * g;
#pragma unroll
          for (int r = 0; r < 4; ++r) sS[vv * LDS_ + c4 + r] = from_f<E>(st[u][nb][r]);
        }
      }
    }
    __syncthreads();
  }

  // ---- final state
#pragma unroll
  for (int u = 0; u < CTW; ++u) {
    const int ct = w * CTW + u;
    if (ct < CT) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        *reinterpret_cast<f32x4 *>(a.S_final + sbase + (size_t)(v0 + 16 * nb + col) * DK + 16 * ct + 4 * g) = st[u][nb];
    }
  }
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
    // value-tile width: enough workgroups to cover the chip
    const long long units = (long long)P.n_seq * a.H;
    int bv = 16;
    if (a.dv >= 64 && units * (a.dv / 64) >= 1024) bv = 64;
    else if (a.dv >= 32 && units * (a.dv / 32) >= 512) bv = 32;
    if (const char *env = std::getenv("KDA_PREFILL_BV")) {
      int b = std::atoi(env);
      if ((b == 16 || b == 32 || b == 64) && b <= a.dv) bv = b;
    }
    const dim3 grid(a.dv / bv, a.H, P.n_seq);
    if (bv == 64)
      hipLaunchKernelGGL((chunk_scan_kernel<DK, 64, E>), grid, dim3(kThreads), 0, stream, sa);
    else if (bv == 32)
      hipLaunchKernelGGL((chunk_scan_kernel<DK, 32, E>), grid, dim3(kThreads), 0, stream, sa);
    else
      hipLaunchKernelGGL((chunk_scan_kernel<DK, 16, E>), grid, dim3(kThreads), 0, stream, sa);
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
