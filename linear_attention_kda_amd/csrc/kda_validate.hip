// kda_validate.hip -- optional device-side checks of the input values that
// the host cannot see (enabled by kda_set_validation or KDA_VALIDATE=1).
//
// The recurrence (page "Kimi Delta Attention (KDA)", opening update
// equation and section "KDA: a separate gate for each key channel") takes
// gates and write strengths in [0, 1] and unit keys (section "DeltaNet:
// writing the error instead of the value": the write removes the old value
// along k exactly when |k| = 1).  A packed batch needs cumulative offsets
// that start at 0, never decrease and end at the token count.  The kernel
// sets one bit per violated condition in a device word; nothing else is
// written.  Grid-stride loops, so any size runs with a fixed grid.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

__device__ unsigned g_validate_bits;

struct ValidateKArgs {
  const float *alpha;
  size_t n_alpha;
  int gate_range;        // 0: in [0, 1]; 1: log gates, <= 0 (-inf allowed); 2: logits, any number
  const float *beta;
  size_t n_beta;
  int beta_logits;       // beta goes through a sigmoid: any number
  const void *k;
  size_t n_krows;        // rows of d_k elements
  int dk, k_bf16;
  const int32_t *cu;
  int n_seq, total;      // cu has n_seq + 1 entries and must end at total
};

template <typename E>
__device__ __forceinline__ float elem(const void *p, size_t i) {
  return (float)reinterpret_cast<const E *>(p)[i];
}

__global__ __launch_bounds__(kThreads) void validate_kernel(ValidateKArgs a) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned bits = 0;
  for (size_t i = tid; i < a.n_alpha; i += stride) {
    const float x = a.alpha[i];
    const bool ok = a.gate_range == 1 ? (x <= 0.f) : a.gate_range == 2 ? (x == x) : (x >= 0.f && x <= 1.f);
    if (!ok) bits |= kValidateAlpha;
  }
  for (size_t i = tid; i < a.n_beta; i += stride) {
    const float x = a.beta[i];
    if (!(x >= 0.f && x <= 1.f) && !(a.beta_logits && x == x)) bits |= kValidateBeta;
  }
  for (size_t r = tid; r < a.n_krows; r += stride) {
    float s = 0.f;
    for (int c = 0; c < a.dk; ++c) {
      const float x = a.k_bf16 ? elem<bf16>(a.k, r * a.dk + c) : elem<float>(a.k, r * a.dk + c);
      s += x * x;
    }
    // unit norm within the rounding of bf16 keys (about 2^-8 relative)
    if (!(fabsf(s - 1.f) <= kValidateKeyTol)) bits |= kValidateKey;
  }
  if (a.cu) {
    for (size_t i = tid; i <= (size_t)a.n_seq; i += stride) {
      const int x = a.cu[i];
      bool ok = x >= 0 && x <= a.total;
      if (i == 0) ok = ok && x == 0;
      if (i == (size_t)a.n_seq) ok = ok && x == a.total;
      if (i > 0) ok = ok && a.cu[i - 1] <= x;
      if (!ok) bits |= kValidateOffsets;
    }
  }
  if (bits) atomicOr(&g_validate_bits, bits);
}

}  // namespace

hipError_t run_validation(const ValidateArgs &v, hipStream_t stream, unsigned *bits) {
  *bits = 0;
  const unsigned zero = 0;
  hipError_t e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_validate_bits), &zero, sizeof(zero), 0,
                                        hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  ValidateKArgs ka{v.alpha, v.n_alpha, v.gate_range, v.beta, v.n_beta, v.beta_logits ? 1 : 0, v.k, v.n_krows, v.dk,
                   v.k_bf16 ? 1 : 0, v.cu, v.n_seq, v.total};
  const size_t work = v.n_alpha > v.n_krows ? v.n_alpha : v.n_krows;
  const unsigned blocks = (unsigned)(work / kThreads + 1 < 4096 ? work / kThreads + 1 : 4096);
  hipLaunchKernelGGL(validate_kernel, dim3(blocks), dim3(kThreads), 0, stream, ka);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbolAsync(bits, HIP_SYMBOL(g_validate_bits), sizeof(unsigned), 0, hipMemcpyDeviceToHost,
                               stream);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(stream);
}

}  // namespace kda
