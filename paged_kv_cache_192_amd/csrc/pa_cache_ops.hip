// Cache-side kernels: slot mapping, the per-token cache write (plain and
// quantising) and the whole-block copy used for copy-on-write and for
// swapping blocks to and from a host pool.  They are bound by launch
// latency at decode batch sizes (the host link for swaps) and never touch
// memory outside the slots or blocks they are given.
#include "pa_internal.h"
#include "pa_quant.h"

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

// Whole-block copy between pools (copy-on-write inside one pool, swap
// between a device and a pinned host pool).  Grid: x = chunk group inside
// a block, y = pair, z = 0 (K) or 1 (V).  Each thread copies kCopyUnroll
// 16-byte chunks of one block, all loads issued before the first store (a
// group that reaches past the block's end takes a guarded path); the
// x = 0 workgroup of each (pair, K/V) also copies the block's scales.
constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

__global__ __launch_bounds__(kCopyThreads) void block_copy_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, const float* __restrict__ src_ks,
    const float* __restrict__ src_vs, uint4* __restrict__ dst_k, uint4* __restrict__ dst_v,
    float* __restrict__ dst_ks, float* __restrict__ dst_vs, const int64_t* __restrict__ pairs,
    int64_t block_chunks, int64_t scales_per_blk, int64_t src_NB, int64_t dst_NB) {
  const int p = blockIdx.y;
  const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= src_NB || dst < 0 || dst >= dst_NB) return;
  const uint4* from = (blockIdx.z ? src_v : src_k) + src * block_chunks;
  uint4* to = (blockIdx.z ? dst_v : dst_k) + dst * block_chunks;
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
  const float* ssc = blockIdx.z ? src_vs : src_ks;
  float* dsc = blockIdx.z ? dst_vs : dst_ks;
  if (ssc && blockIdx.x == 0)
    for (int64_t i = threadIdx.x; i < scales_per_blk; i += kCopyThreads)
      dsc[dst * scales_per_blk + i] = ssc[src * scales_per_blk + i];
}

// ---------------------------------------------------------------------------
// Quantising cache write.  One wave per (token, kv head); lane l holds
// elements l + 64 i of the row (i < D / 64), for K and then V.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_amax(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

template <typename SRC, bool FP8, int PER>
__global__ __launch_bounds__(64) void quantize_and_cache_kernel(
    const SRC* __restrict__ key, const SRC* __restrict__ value, unsigned char* __restrict__ k_cache,
    unsigned char* __restrict__ v_cache, float* __restrict__ k_scales, float* __restrict__ v_scales,
    int per_token, float k_static, float v_static, const int64_t* __restrict__ slots, int Hkv, int BS,
    int64_t num_slots) {
  constexpr int D = 64 * PER;
  const int t = blockIdx.x / Hkv, h = blockIdx.x % Hkv;
  const int lane = threadIdx.x;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t b = slot / BS;
  const int off = (int)(slot % BS);
  const float qmax = quant_max<FP8>();
#pragma unroll
  for (int kv = 0; kv < 2; ++kv) {
    const SRC* src = (kv ? value : key) + ((int64_t)t * Hkv + h) * D;
    float x[PER];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      x[i] = (float)src[lane + 64 * i];
      amax = fmaxf(amax, fabsf(x[i]));
    }
    float s;
    if (per_token) {
      amax = wave_amax(amax);
      s = amax > 0.f ? amax / qmax : 1.f;
    } else {
      s = kv ? v_static : k_static;
    }
    unsigned char* dst = (kv ? v_cache : k_cache) + ((b * Hkv + h) * BS + off) * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      dst[lane + 64 * i] = (unsigned char)quant_code<FP8>(x[i] / s);
    }
    if (lane == 0) {
      float* sc = kv ? v_scales : k_scales;
      sc[per_token ? (b * Hkv + h) * BS + off : b * Hkv + h] = s;
    }
  }
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

pa_status launch_block_copy(const void* src_k, const void* src_v, const float* src_ks, const float* src_vs,
                            void* dst_k, void* dst_v, float* dst_ks, float* dst_vs, int64_t block_bytes,
                            int64_t scales_per_blk, const int64_t* pairs, int32_t P, int32_t src_NB,
                            int32_t dst_NB, hipStream_t st) {
  const int64_t block_chunks = block_bytes / 16;
  const int64_t per_group = (int64_t)kCopyThreads * kCopyUnroll;
  dim3 grid((unsigned)((block_chunks + per_group - 1) / per_group), (unsigned)P, 2);
  hipLaunchKernelGGL(block_copy_kernel, grid, dim3(kCopyThreads), 0, st, (const uint4*)src_k, (const uint4*)src_v,
                     src_ks, src_vs, (uint4*)dst_k, (uint4*)dst_v, dst_ks, dst_vs, pairs, block_chunks,
                     scales_per_blk, (int64_t)src_NB, (int64_t)dst_NB);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "block copy launch");
}

pa_status launch_quantize_and_cache(const void* key, const void* value, pa_dtype src_dtype, void* k_cache,
                                    void* v_cache, pa_dtype kv_dtype, float* k_scales, float* v_scales,
                                    int32_t scale_mode, float k_static, float v_static, const int64_t* slots,
                                    int32_t T, int32_t Hkv, int32_t D, int32_t BS, int32_t NB, hipStream_t st) {
  const size_t waves = (size_t)T * Hkv;
  if (waves > 0x7fffffffu) return fail(PA_ERR_UNSUPPORTED, "pa_quantize_and_cache: grid too large");
  const int per_token = scale_mode == PA_SCALE_TOKEN;
  const int64_t num_slots = (int64_t)NB * BS;
#define PA_QUANT_LAUNCH(SRC, FP8, PER)                                                                         \
  hipLaunchKernelGGL((quantize_and_cache_kernel<SRC, FP8, PER>), dim3((unsigned)waves), dim3(64), 0, st,      \
                     (const SRC*)key, (const SRC*)value, (unsigned char*)k_cache, (unsigned char*)v_cache,    \
                     k_scales, v_scales, per_token, k_static, v_static, slots, Hkv, BS, num_slots)
  const bool fp8 = kv_dtype == PA_FP8_E4M3;
  if (src_dtype == PA_F32) {
    if (fp8) { if (D == 64) PA_QUANT_LAUNCH(float, true, 1); else PA_QUANT_LAUNCH(float, true, 2); }
    else { if (D == 64) PA_QUANT_LAUNCH(float, false, 1); else PA_QUANT_LAUNCH(float, false, 2); }
  } else {
    if (fp8) { if (D == 64) PA_QUANT_LAUNCH(__bf16, true, 1); else PA_QUANT_LAUNCH(__bf16, true, 2); }
    else { if (D == 64) PA_QUANT_LAUNCH(__bf16, false, 1); else PA_QUANT_LAUNCH(__bf16, false, 2); }
  }
#undef PA_QUANT_LAUNCH
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_quantize_and_cache launch");
}

}  // namespace pa
