// rla2_fwd_chunked_noalloc: the chunked forward with its workspace in a file-scope device array
// instead of a caller buffer, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array `scratch` exists once per GPU the library runs on and is held until the process
// ends. In host code its name is only a host-side stand-in: its device address is looked up
// with hipGetSymbolAddress once per device (with that device current, on the first call on
// it) and only that address is ever handed to the kernels. Every call on a GPU shares the
// GPU's array, so calls that overlap on one GPU (other streams, other threads) race on it.
// The forward needs no part of its workspace cleared on entry (its set-up launch writes the
// tables and the status header, the state pass every record it reads later).
#include <hip/hip_runtime.h>

#include <mutex>

#include "rla2.h"
#include "rla2_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)RLA2_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the first call there).
rla2_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RLA2_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RLA2_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return RLA2_ERR_HIP;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return RLA2_OK;
}

}  // namespace

extern "C" rla2_status rla2_fwd_chunked_noalloc(const rla2_fwd_desc* desc, const void* q, const void* k,
                                                const void* v, const float* gamma_q, const float* gamma_k,
                                                void* out, float* final_S, float* final_z, hipStream_t stream) {
  size_t need = 0;
  rla2_status st = rla2_fwd_workspace_size(desc, &need);
  if (st != RLA2_OK) return st;
  if (need > kScratchBytes) return RLA2_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != RLA2_OK) return st;
  return rla2_fwd_chunked(desc, q, k, v, gamma_q, gamma_k, out, final_S, final_z, ws, kScratchBytes, stream);
}
