// Internal declarations shared by the host API (pa_api.cpp) and the kernel
// translation units.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

// Records a message for pa_last_error() on the calling thread and returns s.
pa_status fail(pa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status hip_fail(hipError_t e, const char* what);

inline int dtype_bytes(pa_dtype t) {
  switch (t) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_I8: return 1;
  }
  return 0;
}

// ---- decode planning -----------------------------------------------------

enum KernelKind { KERNEL_VALU = 1, KERNEL_MFMA = 2 };

// Everything the launchers need, derived on the host from pa_decode_args.
struct DecodePlan {
  KernelKind kind;
  int G;                 // query heads per kv head
  int heads_per_wave;    // VALU: heads handled by one wave (1, 2, 4 or 8)
  int head_groups;       // VALU: ceil(G / heads_per_wave)
  int partition_tokens;  // multiple of 16
  int num_partitions;    // ceil(max_context_len / partition_tokens), >= 1
  size_t workspace_bytes;
};

pa_status plan_decode(const pa_decode_args* a, DecodePlan* plan);

// Workspace layout for num_partitions > 1:
//   float2 ml [S][Hq][nP]        (running max in log2 units, sum of weights)
//   float  acc[S][Hq][nP][D]     (unnormalised weighted sum of values)
inline size_t ws_ml_bytes(int S, int Hq, int nP) {
  size_t b = (size_t)S * Hq * nP * 2 * sizeof(float);
  return (b + 255) & ~(size_t)255;
}

pa_status launch_decode_mfma(const pa_decode_args* a, const DecodePlan& p, hipStream_t st);
pa_status launch_decode_valu(const pa_decode_args* a, const DecodePlan& p, hipStream_t st);
pa_status launch_decode_reduce(const pa_decode_args* a, const DecodePlan& p, hipStream_t st);

pa_status launch_slot_mapping(const int32_t* block_tables, int32_t max_blocks, int32_t num_seqs, const int32_t* seq_idx,
                              const int32_t* positions, const int32_t* context_lens, int32_t T,
                              int32_t BS, int64_t* slots, hipStream_t st);
pa_status launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                   int elem_bytes, const int64_t* slots, int32_t T, int32_t Hkv,
                                   int32_t D, int32_t BS, int32_t NB, hipStream_t st);
pa_status launch_copy_blocks(void* k_cache, void* v_cache, int elem_bytes, float* k_scales,
                             float* v_scales, const int64_t* pairs, int32_t P, int32_t Hkv, int32_t D,
                             int32_t BS, int32_t NB, hipStream_t st);

}  // namespace pa
