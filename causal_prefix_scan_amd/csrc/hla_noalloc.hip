// hla_fwd_noalloc: the chunk-parallel forward (hla_fwd) for callers that
// cannot allocate device memory (code under graph capture, tight serving
// loops, harnesses that forbid allocation).  Its workspace -- the segment
// summaries and the scan's scratch -- lives in a file-scope device array of
// fixed size instead of a caller buffer; the kernels are the same ones hla_fwd
// launches, and they take the array's device address as their buffer.
//
// Each device that runs this entry point holds its own copy of the array, at
// its own address, until the process ends.  That address is looked up once
// per device, with the device current, and kept; host code never passes the
// array's name itself to a kernel or a copy (in host code the name is only a
// host-side stand-in).
#include <hip/hip_runtime.h>

#include <mutex>

#include "hla.h"
#include "hla_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's copy of `scratch`, looked up on first use.
hla_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return HLA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return HLA_ERR_HIP;
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return HLA_OK;
}

}  // namespace

extern "C" {

size_t hla_fwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

hla_status hla_fwd_noalloc(const hla_problem* p, const void* q, const void* k, const void* v,
                           float* o, float* den, const hla_state* final_state,
                           void* stream) try {
  // every argument check of hla_fwd, before any HIP call
  if (hla_status e = hla::fwd_validate(p, q, k, v, o, den, final_state, nullptr, 0, false))
    return e;
  if (p->B == 0 || p->H == 0 || p->T == 0) return HLA_OK;
  const size_t need = hla_fwd_workspace_bytes(p);
  if (need > kScratchBytes) return HLA_ERR_WORKSPACE_TOO_SMALL;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return HLA_ERR_HIP;
  }
  void* ws = nullptr;
  if (hla_status e = scratch_on_current_device(&ws)) return e;
  return hla::fwd_enqueue(p, q, k, v, o, den, final_state, ws, need, stream);
} catch (...) {
  return HLA_ERR_HIP;
}

}  // extern "C"
