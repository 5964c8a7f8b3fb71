// Cache-side kernels: slot mapping, the per-token cache write and the
// copy-on-write block copy.  All three are byte movers bound by launch
// latency at decode batch sizes; they use 16-byte vector accesses and never
// touch memory outside the slots or blocks they are given.
#include "pa_internal.h"

namespace pa {

// slot = table[seq][pos / BS] * BS + pos % BS (glossary figure, section 2:
// logical block -> physical block through the table).  -1 when the position
// or the table entry is unusable.
__global__ void slot_mapping_kernel(const int32_t* __restrict__ tables, int32_t max_blocks, int32_t num_seqs,
                                    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ positions,
                                    const int32_t* __restrict__ context_lens, int32_t T, int32_t BS,
                                    int64_t* __restrict__ slots) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int seq = seq_idx ? seq_idx[t] : t;
  int64_t slot = -1;
  if (seq < 0 || seq >= num_seqs) {
    slots[t] = slot;
    return;
  }
  const int pos = positions ? positions[t] : context_lens[seq] - 1;
  if (pos >= 0 && pos / BS < max_blocks) {
    const int32_t b = tables[(int64_t)seq * max_blocks + pos / BS];
    if (b >= 0) slot = (int64_t)b * BS + pos % BS;
  }
  slots[t] = slot;
}

// One block of threads per new token; each thread moves 16-byte chunks of
// the token's [Hkv][D] key and value rows into cache[slot/BS][h][slot%BS][:].
// row_chunks = Hkv * D * elem / 16, head_chunks = D * elem / 16.
__global__ void reshape_and_cache_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                                         uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                         const int64_t* __restrict__ slots, int32_t row_chunks,
                                         int32_t head_chunks, int32_t BS, int64_t num_slots) {
  const int t = blockIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t b = slot / BS;
  const int off = (int)(slot % BS);
  for (int c = threadIdx.x; c < row_chunks; c += blockDim.x) {
    const int h = c / head_chunks;
    const int w = c % head_chunks;
    const int64_t dst = ((b * (row_chunks / head_chunks) + h) * BS + off) * head_chunks + w;
    const int64_t src = (int64_t)t * row_chunks + c;
    k_cache[dst] = key[src];
    v_cache[dst] = value[src];
  }
}

// Grid: x = chunk group inside a block, y = pair, z = 0 (K) or 1 (V).
// Each thread copies kCopyUnroll 16-byte chunks of one physical block, all
// loads issued before the first store (a group that reaches past the
// block's end takes a guarded path); the first threads of each (pair, K/V)
// also copy that block's per-head scales when present.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    uint4* __restrict__ k_cache, uint4* __restrict__ v_cache, float* __restrict__ k_scales,
    float* __restrict__ v_scales, const int64_t* __restrict__ pairs, int64_t block_chunks, int32_t Hkv,
    int64_t num_blocks) {
  const int p = blockIdx.y;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* cache = blockIdx.z ? v_cache : k_cache;
  const uint4* from = cache + src * block_chunks;
  uint4* to = cache + dst * block_chunks;
  const int64_t group = (int64_t)blockIdx.x * kCopyThreads * kCopyUnroll;
  const int64_t base = group + threadIdx.x;
  if (group + kCopyThreads * kCopyUnroll <= block_chunks) {
    const uint4 a = from[base], b = from[base + kCopyThreads];
    const uint4 c = from[base + 2 * kCopyThreads], d = from[base + 3 * kCopyThreads];
    to[base] = a;
    to[base + kCopyThreads] = b;
    to[base + 2 * kCopyThreads] = c;
    to[base + 3 * kCopyThreads] = d;
  } else {
    for (int64_t i = base; i < block_chunks; i += kCopyThreads) to[i] = from[i];
  }
  float* scales = blockIdx.z ? v_scales : k_scales;
  if (scales && blockIdx.x == 0 && threadIdx.x < Hkv) scales[dst * Hkv + threadIdx.x] = scales[src * Hkv + threadIdx.x];
}

pa_status launch_slot_mapping(const int32_t* block_tables, int32_t max_blocks, int32_t num_seqs, const int32_t* seq_idx,
                              const int32_t* positions, const int32_t* context_lens, int32_t T, int32_t BS,
                              int64_t* slots, hipStream_t st) {
  const int threads = 256;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((T + threads - 1) / threads), dim3(threads), 0, st, block_tables,
                     max_blocks, num_seqs, seq_idx, positions, context_lens, T, BS, slots);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_slot_mapping launch");
}

pa_status launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                   int elem_bytes, const int64_t* slots, int32_t T, int32_t Hkv, int32_t D,
                                   int32_t BS, int32_t NB, hipStream_t st) {
  const int head_chunks = D * elem_bytes / 16;
  const int row_chunks = Hkv * head_chunks;
  int threads = row_chunks < 256 ? ((row_chunks + 63) / 64) * 64 : 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(T), dim3(threads), 0, st, (const uint4*)key,
                     (const uint4*)value, (uint4*)k_cache, (uint4*)v_cache, slots, row_chunks, head_chunks, BS,
                     (int64_t)NB * BS);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_reshape_and_cache launch");
}

pa_status launch_copy_blocks(void* k_cache, void* v_cache, int elem_bytes, float* k_scales, float* v_scales,
                             const int64_t* pairs, int32_t P, int32_t Hkv, int32_t D, int32_t BS,
                             int32_t NB, hipStream_t st) {
  const int64_t block_chunks = (int64_t)Hkv * BS * D * elem_bytes / 16;
  const int64_t per_group = (int64_t)kCopyThreads * kCopyUnroll;
  dim3 grid((unsigned)((block_chunks + per_group - 1) / per_group), (unsigned)P, 2);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(kCopyThreads), 0, st, (uint4*)k_cache, (uint4*)v_cache, k_scales,
                     v_scales, pairs, block_chunks, Hkv, (int64_t)NB);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_copy_blocks launch");
}

}  // namespace pa
