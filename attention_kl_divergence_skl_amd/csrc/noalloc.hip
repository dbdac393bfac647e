// Allocation-free split-K forward: the partials live in a file-scope device
// array (one copy per GPU, held for the life of the process) instead of a
// caller workspace, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// The array's name is a host-side stand-in in host code; the device address
// of each GPU's copy is looked up once per device with hipGetSymbolAddress and
// only that address is passed on.  Every call on a GPU shares that GPU's
// array: calls that overlap on one GPU (two streams, two host threads) race.
// Nothing needs clearing: the split kernel writes every (row, split) partial,
// empty splits included, before the reduce reads it.

#include <mutex>

#include "../../include/streamkl.h"
#include "skl_internal.h"

namespace skl {

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch` (nullptr on failure).
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace skl

extern "C" {

size_t skl_noalloc_scratch_bytes(void) { return skl::kScratchBytes; }

skl_status skl_forward_splitk_noalloc(const skl_shape* shape, const void* q1, const void* k1, const void* q2,
                                      const void* k2, float scale1, float scale2, int causal, int num_splits,
                                      float* kl, float* lse1, float* lse2, hipStream_t stream) {
  // Host checks first (no HIP call): the partials must fit the array.
  if (shape && num_splits >= 1) {
    const size_t need = skl_forward_splitk_workspace_size(shape, num_splits);
    if (need > skl::kScratchBytes)
      return skl::set_error(SKL_ERR_UNSUPPORTED,
                            "skl_forward_splitk_noalloc: the partials need %zu bytes, more than the %zu-byte "
                            "static scratch array (B * H * N_Q * num_splits * 20 bytes)",
                            need, skl::kScratchBytes);
  }
  void* ws = nullptr;
  const hipError_t e = skl::scratch_for_current_device(&ws);
  if (e != hipSuccess)
    return skl::set_error(SKL_ERR_HIP, "skl_forward_splitk_noalloc: scratch address: %s", hipGetErrorString(e));
  const skl_status st = skl_forward_splitk(shape, q1, k1, q2, k2, scale1, scale2, causal, num_splits, ws,
                                           skl::kScratchBytes, stream);
  if (st != SKL_OK) return st;
  return skl_reduce(shape, num_splits, ws, skl::kScratchBytes, kl, lse1, lse2, stream);
}

}  // extern "C"
