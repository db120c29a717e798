// Forward-only entry point that allocates nothing: the scratch of the
// inference forward (esg_sparse_swiglu_fwd with saved = NULL) comes from a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// Each device the library runs on holds its own copy of the array until the
// process ends.  Its device address is taken once per device, with that device
// current, by hipGetSymbolAddress; host code only ever passes that address to
// the kernels (the array's name is a host-side stand-in, not a device address).
// Calls on one device share the array: the last call's contents stay in it,
// and calls that overlap on one device (two streams, two threads) race.  The
// forward needs nothing cleared: every scratch word it reads was written
// earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "esg.h"
#include "esg_internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)ESG_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

// per-device address of `scratch`, or nullptr before the first lookup
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ESG_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ESG_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ESG_OK;
}

}  // namespace

extern "C" int esg_sparse_swiglu_fwd_noalloc(const void* x, const void* w_gate, const void* w_up,
                                             const void* w_down, int dtype, int tokens, int d_model, int d_ff,
                                             int group_size, int k, const int32_t* idx, void* y,
                                             int32_t* status_dev, void* stream) {
  // validates the shape (and, for idx = NULL, rejects the dense limit's k)
  int st = esg_sparse_swiglu_workspace_size(tokens, d_model, d_ff, group_size, k, dtype, idx == nullptr, nullptr,
                                            nullptr, nullptr);
  if (st != ESG_OK) return st;
  const esg::FfnShape s{dtype, tokens, d_model, d_ff, group_size, k};
  const size_t fwd_bytes = idx == nullptr ? 0 : esg::inference_fwd_scratch_bytes(s);
  if (fwd_bytes > kScratchBytes) return ESG_ERR_WORKSPACE;
  void* ptr = nullptr;
  st = scratch_ptr(&ptr);
  if (st != ESG_OK) return st;
  return esg_sparse_swiglu_fwd(x, w_gate, w_up, w_down, dtype, tokens, d_model, d_ff, group_size, k, idx, y,
                               nullptr, 0, ptr, kScratchBytes, status_dev, stream);
}
