// host_stubs.cpp -- host-only stand-ins for the kernel launchers and for the
// three HIP runtime calls that kda_api.cpp makes, so the C ABI's argument
// checks and workspace planning can be built with the address and
// undefined-behaviour sanitizers and run on a machine without a GPU.  Test
// infrastructure only: never linked into libkda.so.
//
// The launch stand-ins check that what the ABI layer hands the launchers is
// consistent (the workspace plan fits the workspace it was checked against,
// the shapes are the ones the call was made with) and count the calls; the
// counts are read back through kda_stub_calls().
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "kda_launch.h"

namespace {
int g_calls[3];        // prefill, decode, validation
int g_bad_plans;       // plans that failed a consistency check
bool g_last_decode_module;  // the last decode launch carried a module operation
}  // namespace

namespace kda {

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t) {
  ++g_calls[0];
  const WorkspacePlan &P = a.plan;
  // the split-sequence buffers, when planned, follow the ready flags in order
  const size_t base_end = P.ready + P.ready_bytes;
  const size_t state = (size_t)a.dv * a.dk * sizeof(float);
  const bool split_ok =
      P.split.G > 1 ? (!a.cu_seqlens && P.sp_tables == base_end && P.sp_maps > P.sp_tables &&
                       P.sp_start == P.sp_maps + (size_t)a.B * (P.split.G - 1) * a.H * (a.dv + a.dk) * a.dk * 4 &&
                       P.sp_end == P.sp_start + (size_t)a.B * P.split.G * a.H * state &&
                       P.total == P.sp_end + (size_t)a.B * P.split.G * a.H * state &&
                       (long long)P.split.cps * (P.split.G - 1) < ((long long)a.T + 63) / 64)
                    : P.total == base_end;
  const bool ok = P.tables == kCtlBytes && P.records == P.tables + P.tables_bytes &&
                  P.ready == P.records + (size_t)P.max_chunks * a.H * P.record_bytes &&
                  split_ok && P.record_bytes % 1024 == 0 && a.ws != nullptr &&
                  (a.cu_seqlens ? P.ready_bytes == 0 : P.n_seq == a.B) && a.scale > 0.f &&
                  (a.dk == 16 || a.dk == 32 || a.dk == 64 || a.dk == 128);
  if (!ok) ++g_bad_plans;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t) {
  ++g_calls[1];
  if (a.N <= 0 || a.H <= 0 || a.Tk < 0 || !a.S || !a.S_in || a.scale <= 0.f) ++g_bad_plans;
  // the module operations: all convolution pointers or none
  const bool any_conv = a.conv_q || a.conv_k || a.conv_v || a.conv_state;
  if (any_conv && !(a.conv_q && a.conv_k && a.conv_v && a.conv_state)) ++g_bad_plans;
  g_last_decode_module = any_conv || a.norm_w || a.out_gate;
  return hipSuccess;
}

hipError_t run_validation(const ValidateArgs &, hipStream_t, unsigned *bits) {
  ++g_calls[2];
  *bits = 0;
  return hipSuccess;
}

void release_overlap() {}

// a fake but aligned device address (never dereferenced: the launches above
// are stand-ins too)
hipError_t scratch_address(void **ptr) {
  *ptr = reinterpret_cast<void *>((uintptr_t)1 << 44);
  return hipSuccess;
}

}  // namespace kda

extern "C" {

// which: 0 prefill launches, 1 decode launches, 2 validation runs, 3 plans
// that failed a consistency check, 4 whether the last decode launch carried
// a module operation; -1 resets every count
int kda_stub_calls(int which) {
  if (which < 0) {
    std::memset(g_calls, 0, sizeof(g_calls));
    g_bad_plans = 0;
    g_last_decode_module = false;
    return 0;
  }
  if (which == 4) return g_last_decode_module ? 1 : 0;
  return which < 3 ? g_calls[which] : g_bad_plans;
}

hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus *s) {
  *s = hipStreamCaptureStatusNone;
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void *dst, const void *, size_t n, hipMemcpyKind, hipStream_t) {
  std::memset(dst, 0, n);  // no device: the status words read back as zero
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }

}  // extern "C"
