// static_step.hip — clsa_decode_step_static: the decode step running on the
// library's own device scratch instead of a caller-provided workspace, for
// callers that cannot allocate device memory (work recorded under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The scratch is one file-scope device array of kScratchBytes per GPU,
// resident from the module's load on that GPU until the process ends. Its
// device address is looked up once per device (with that device current) and
// kept; host code never uses the array's own name as an address. Every call
// on a GPU shares that GPU's array: calls that overlap in time on one GPU
// (two streams, two threads) race on it. The step's kernels write every
// scratch word they later read (top-k chunk counts and candidate segments,
// attention split states, indexer scores, kept counts), so no call depends on
// what the previous call left behind.
#include <mutex>

#include "kernels.h"

namespace clsa {
namespace {

constexpr size_t kScratchBytes = CLSA_STATIC_SCRATCH_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device

// Device address of this device's scratch, looked up on the first call on the
// device (the device is current).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(CLSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(CLSA_ERR_UNSUPPORTED, "decode_step_static: device %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(CLSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CLSA_OK;
}

}  // namespace
}  // namespace clsa

using namespace clsa;

extern "C" {

int clsa_decode_step_static(const clsa_step_desc* d, void* stream) {
  const size_t need = clsa_decode_step_workspace_bytes(d);
  if (need == 0)  // invalid descriptor: the regular entry point reports why, launching nothing
    return clsa_decode_step(d, nullptr, 0, stream);
  if (need > kScratchBytes)
    return set_error(CLSA_ERR_WORKSPACE,
                     "decode_step_static: the step needs %zu bytes of scratch, above the library's "
                     "%zu (use clsa_decode_step with a caller workspace)",
                     need, kScratchBytes);
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  return clsa_decode_step(d, ws, kScratchBytes, stream);
}

}  // extern "C"
