// Read-bandwidth probe: the memory system's ceiling for the reads decode
// does.  Decode attention streams every cached byte once per step, in
// chunks of one (block, kv head) -- 4 KiB for 16 tokens of 128 bf16 values,
// 2 KiB with 1-byte codes -- scattered by the block tables (glossary "PagedAttention & Gestion du
// KV-Cache", section 2 figure).  This kernel reads 4 KiB chunks and nothing
// else: in address order (the plain streaming ceiling) or in the order of a
// given list of chunk ids (the decode's table order), with the same
// 16-byte non-temporal loads, so a decode kernel's rate can be compared
// with what a read alone achieves on the same bytes.  Not part of
// attention; diagnostic only.
#include "pa_internal.h"

namespace pa {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Wave w reads chunks w, w + W, w + 2W, ... of CHUNK bytes (1, 2 or 4 KiB:
// one 16-byte load per lane per KiB), two at a time (both chunks' loads
// issued before either is consumed); each lane folds what it read into one
// word, stored to sink[w * 64 + lane] so the loads stay live.
template <int CHUNK>
__global__ __launch_bounds__(64) void read_probe_kernel(const char* __restrict__ base,
                                                        const int32_t* __restrict__ ids, int64_t n,
                                                        unsigned* __restrict__ sink) {
  constexpr int LOADS = CHUNK / (64 * 16);
  const int lane = threadIdx.x;
  const int64_t W = gridDim.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t c = blockIdx.x; c < n; c += 2 * W) {
    const int64_t c1 = c + W < n ? c + W : c;
    const int64_t i0 = ids ? ids[c] : c, i1 = ids ? ids[c1] : c1;
    const char* p0 = base + i0 * CHUNK + lane * 16;
    const char* p1 = base + i1 * CHUNK + lane * 16;
    u32x4_t a[LOADS], b[LOADS];
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      a[k] = __builtin_nontemporal_load((const u32x4_t*)(p0 + k * 1024));
      b[k] = __builtin_nontemporal_load((const u32x4_t*)(p1 + k * 1024));
    }
#pragma unroll
    for (int k = 0; k < LOADS; ++k) acc ^= a[k] ^ b[k];
  }
  sink[blockIdx.x * 64 + lane] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace pa

using namespace pa;

extern "C" {

pa_status pa_read_probe(const void* base, int64_t num_chunks, const int32_t* chunk_ids, int32_t chunk_bytes,
                        int32_t num_waves, uint32_t* sink, void* stream) {
  if (num_chunks < 0 || num_waves <= 0)
    return fail(PA_ERR_INVALID, "pa_read_probe: num_chunks must be >= 0 and num_waves > 0");
  if (chunk_bytes != 1024 && chunk_bytes != 2048 && chunk_bytes != 4096)
    return fail(PA_ERR_INVALID, "pa_read_probe: chunk_bytes %d not in {1024, 2048, 4096}", chunk_bytes);
  if (num_chunks == 0) return PA_OK;
  if (!base || !sink) return fail(PA_ERR_INVALID, "pa_read_probe: NULL device pointer");
  if ((uintptr_t)base % 16 || (uintptr_t)sink % 4 || (chunk_ids && (uintptr_t)chunk_ids % 4))
    return fail(PA_ERR_INVALID, "pa_read_probe: base must be 16-byte aligned, sink and chunk_ids 4-byte");
#define PA_PROBE_LAUNCH(C)                                                                                     \
  hipLaunchKernelGGL(read_probe_kernel<C>, dim3((unsigned)num_waves), dim3(64), 0, (hipStream_t)stream,        \
                     (const char*)base, chunk_ids, num_chunks, (unsigned*)sink)
  if (chunk_bytes == 1024) PA_PROBE_LAUNCH(1024);
  else if (chunk_bytes == 2048) PA_PROBE_LAUNCH(2048);
  else PA_PROBE_LAUNCH(4096);
#undef PA_PROBE_LAUNCH
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_read_probe launch");
}

}  // extern "C"
