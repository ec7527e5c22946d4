// hyperattn_forward without a caller workspace, for callers that cannot
// allocate device memory (code under stream capture, serving loops, hosts
// that forbid allocation): the workspace is a fixed array in the library's
// device code object, one per GPU, held until the process ends.
//
// The array's host-side name is not a device address; its address on the
// current device comes from hipGetSymbolAddress, taken once per device on
// that device's first call and kept. Every call on one GPU shares that GPU's
// array, so calls that overlap on one GPU race; the forward pass reads no
// workspace byte it has not written in the same call (its work-queue
// counters are zeroed by a kernel), so what an earlier call left there does
// not matter.
#include <mutex>

#include "common.h"

namespace ha {

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = 0;
  HA_HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HA_ERR_UNSUPPORTED, "device %d is beyond the %d this entry point serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    HA_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(HA_ERR_HIP, "hipGetSymbolAddress returned no address for the scratch");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return HA_OK;
}

}  // namespace

}  // namespace ha

using namespace ha;

extern "C" {

size_t hyperattn_noalloc_scratch_bytes(void) { return kScratchBytes; }

int hyperattn_forward_noalloc(const void* Q, const void* K, const void* V, void* O, float* lse,
                              int64_t n, int d, int heads, int causal, int b, int m,
                              int recursion_base, int r, uint64_t seed, int dtype, void* stream) {
  set_error("%s", "");
  Plan p;
  int rc = make_plan(p, n, d, heads, causal, b, m, recursion_base, r, dtype, true);
  if (rc != HA_OK) return rc;
  if (p.total > kScratchBytes)
    return fail(HA_ERR_WORKSPACE,
                "these sizes need %zu bytes of workspace; the static scratch holds %zu "
                "(use hyperattn_forward with a caller workspace)",
                p.total, kScratchBytes);
  if (n == 0 || heads == 0) return HA_OK;
  if (!Q || !K || !V || !O) return fail(HA_ERR_NULL, "Q, K, V and O must not be NULL");
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != HA_OK) return rc;
  return hyperattn_forward(Q, K, V, O, lse, n, d, heads, causal, b, m, recursion_base, r, seed,
                           dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
