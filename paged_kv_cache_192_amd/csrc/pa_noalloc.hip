// pa_decode_noalloc: decode attention whose split-K workspace is a fixed
// array owned by the library, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  Same plan, same kernels and same result as
// pa_decode with a caller-owned workspace.
//
// The array below is a device global: every GPU the library runs on holds
// its own copy, at its own address, from the module's load until the
// process ends.  In host code its name is only a stand-in; the device
// address is asked for once per device (hipGetSymbolAddress, with that
// device current) and kept.  Every call on one GPU shares that GPU's copy:
// calls that may overlap on one GPU (two streams, two threads) race.  The
// workspace needs no clearing: every partial the merge reads is written by
// the same call.
#include <mutex>

#include "pa_internal.h"

namespace pa {

constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the
// first call made with that device current).
static pa_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "pa_decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_noalloc: device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "pa_decode_noalloc: hipGetSymbolAddress");
    if (!p) return fail(PA_ERR_HIP, "pa_decode_noalloc: hipGetSymbolAddress returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" {

size_t pa_decode_noalloc_scratch_bytes(void) { return kNoallocScratchBytes; }

pa_status pa_decode_noalloc(const pa_decode_args* a) {
  DecodePlan p;
  pa_status s = plan_decode(a, &p);
  if (s != PA_OK) return s;
  if (p.workspace_bytes > kNoallocScratchBytes)
    return fail(PA_ERR_INVALID,
                "pa_decode_noalloc: these arguments need %zu bytes of workspace; the library's fixed scratch holds "
                "%zu (use pa_decode with a caller-owned workspace)",
                p.workspace_bytes, kNoallocScratchBytes);
  if (a->num_seqs == 0) return PA_OK;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != PA_OK) return s;
  pa_decode_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = kNoallocScratchBytes;
  return pa_decode(&b);
}

}  // extern "C"
