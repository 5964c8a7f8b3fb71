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

// Checks of the device-side preconditions pa.h leaves to the caller, when
// the environment variable PA_DEBUG is set (pa_debug.cpp).
bool debug_enabled();
pa_status debug_check_decode(const pa_decode_args* a, hipStream_t st);
pa_status debug_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                            hipStream_t st, const char* fn);
pa_status debug_check_pairs(const int64_t* block_pairs, int32_t num_pairs, int32_t src_num_blocks,
                            int32_t dst_num_blocks, bool same_pool, hipStream_t st, const char* fn);

inline int dtype_bytes(pa_dtype t) {
  switch (t) {
    case PA_F32: return 4;
    case PA_BF16: return 2;
    case PA_I8: return 1;
    case PA_FP8_E4M3: return 1;
  }
  return 0;
}

// int8 and E4M3 caches carry fp32 scales.
inline bool quantised(pa_dtype t) { return t == PA_I8 || t == PA_FP8_E4M3; }

// fp32 scales per physical block (all kv heads) in a scale layout.
inline int64_t scales_per_block(int32_t mode, int32_t Hkv, int32_t BS) {
  return mode == PA_SCALE_TOKEN ? (int64_t)Hkv * BS : (int64_t)Hkv;
}

// ---- decode planning -----------------------------------------------------

enum KernelKind { KERNEL_VALU = 1, KERNEL_MFMA = 2 };

// Longest partition, in blocks: the matrix-core kernel keeps a partition's
// table entries in two registers of 64 lanes.
constexpr int kMaxPartitionBlocks = 128;
// Most partitions the automatic plan splits one sequence into: for a batch
// of near-equal lengths, and for a ragged batch (where it bounds the
// workspace, which holds max_context_len / partition_tokens partials per
// row).
constexpr int kMaxAutoPartitions = 32;
// waves per work item of the shared-prefix (cascade) decode
constexpr int kCascadeWaves = 4;
// balanced split of a ragged batch: at most this many sequences (the
// lengths sit in four 64-lane chunks of registers; sixteen chunks, up to
// kBalancedWideMaxSeqs, in the wide form) and tiles per wave range
constexpr int kBalancedMaxSeqs = 256;
constexpr int kBalancedWideMaxSeqs = 1024;
constexpr int kBalancedMaxTiles = 64;
constexpr int kMaxRaggedPartitions = 512;
// Most partitions one workgroup takes in a grouped launch (one wave each,
// combined through LDS: 2, 4 or 8 waves)
constexpr int kMaxGroupWaves = 8;
// ... and only with at least this many (sequence, kv head) items: one
// workgroup per compute unit of the chip
constexpr int64_t kGroupMinItems = 256;
// An automatic split into more partitions than a group holds is still
// grouped (4 waves) when the longest sequence has at most this many tiles
constexpr int64_t kGroupShortTiles = 128;
// ... and a batch of at most this many tiles in all takes at most 4 waves
// per group
constexpr int64_t kGroupSmallTiles = 16384;
// waves of a workgroup sharing K/V tiles through LDS (several query rows
// per sequence, head_dim 128, more than one wave of column groups per
// item), one column group each: registers for 4 waves per SIMD
constexpr int kSharedWaves = 16;

// Everything the launchers need, derived on the host from pa_decode_args.
struct DecodePlan {
  KernelKind kind;
  int G;                 // query heads per kv head
  int heads_per_wave;    // VALU: heads handled by one wave (1, 2, 4 or 8)
  int head_groups;       // VALU: ceil(G / heads_per_wave)
  int partition_tokens;  // multiple of 16
  int num_partitions;    // ceil(max_context_len / partition_tokens), >= 1
  int cgroups;           // MFMA: groups of 16 (query row, head) columns per (sequence, kv head)
  int ncg;               // MFMA: column groups carried by one wave (1 or 2)
  int cg_waves;          // MFMA: waves per (sequence, kv head, partition) = ceil(cgroups / ncg)
  bool shared_tiles;     // MFMA, several query rows: the waves of a workgroup share each K/V tile
  int64_t rows;          // output rows: query rows (num_seqs, or num_queries) x num_q_heads
  // shared prefix (cascade): items over the shared blocks for all
  // sequences, split into prefix_partitions partitions of prefix_tokens,
  // with prefix_cgroups column groups (sequences x heads, 16 at a time,
  // one wave each); the per-sequence items then start at the prefix's end
  bool cascade;
  int prefix_tokens, prefix_partitions, prefix_cgroups;
  int ws_partitions;     // partials per output row: prefix_partitions + num_partitions
  // balanced split (ragged batch): each kv head's tiles, in sequence order,
  // cut into equal ranges of at least balanced_min_tiles, one per wave of
  // balanced_waves per head; ws_partitions partial slots per row
  bool balanced;
  int balanced_waves, balanced_min_tiles;
  // groups (MFMA, one column group per item, 2 .. kMaxGroupWaves
  // partitions, no cascade or balanced split): one workgroup of group_waves
  // waves per (sequence, kv head), wave w on partition w, combined through
  // LDS; no partials (ws_partitions = 1)
  bool grouped;
  int group_waves;
  size_t workspace_bytes;
};

pa_status plan_decode(const pa_decode_args* a, DecodePlan* plan);

// Workspace layout for ws_partitions > 1 (offsets 256-byte aligned), with
// nP = ws_partitions (shared-prefix partials first, then the sequences'):
//   float2 ml [rows][nP]      reference max (log2 units), sum of weights
//   float  acc[rows][nP][D]   unnormalised weighted sum of values
// Every entry a merge reads is written by the same call, so the workspace
// needs no initialisation.
struct WorkspaceLayout {
  size_t ml_offset, acc_offset, counts_offset, out_offset, bytes;
};

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

inline WorkspaceLayout workspace_layout(const pa_decode_args* a, const DecodePlan& p) {
  WorkspaceLayout L{0, 0, 0, 0, 0};
  if (p.ws_partitions > 1) {
    const size_t rows = (size_t)p.rows * p.ws_partitions;
    L.ml_offset = 0;
    L.acc_offset = align256(rows * 2 * sizeof(float));
    L.counts_offset = L.acc_offset + align256(rows * a->head_dim * sizeof(float));
    // balanced split: partials per sequence, int32 [num_seqs]
    L.bytes = L.counts_offset + (p.balanced ? align256((size_t)a->num_seqs * sizeof(int32_t)) : 0);
  }
  // a bf16 output: the fp32 result rows, rounded into out by a last pass
  if (a->out_dtype == PA_BF16) {
    L.out_offset = L.bytes;
    L.bytes += align256((size_t)p.rows * a->head_dim * sizeof(float));
  }
  return L;
}

pa_status launch_decode_mfma(const pa_decode_args* a, const DecodePlan& p, hipStream_t st);
pa_status launch_decode_valu(const pa_decode_args* a, const DecodePlan& p, hipStream_t st);
pa_status launch_decode_merge(const pa_decode_args* a, const DecodePlan& p, hipStream_t st);
// n fp32 values -> bf16, round to nearest even (n a multiple of 4)
pa_status launch_f32_to_bf16(const float* in, void* out, size_t n, hipStream_t st);

pa_status launch_slot_mapping(const int32_t* block_tables, int32_t max_blocks, int32_t num_seqs, const int32_t* seq_idx,
                              const int32_t* positions, const int32_t* context_lens, int32_t T,
                              int32_t BS, int64_t* slots, hipStream_t st);
pa_status launch_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                                   int elem_bytes, const int64_t* slots, int32_t T, int32_t Hkv,
                                   int32_t D, int32_t BS, int32_t NB, hipStream_t st);
// Whole-block copies from pool `src` to pool `dst` (the same pool for
// copy-on-write); scales_per_blk fp32 scales follow each block when given.
pa_status launch_block_copy(const void* src_k, const void* src_v, const float* src_ks, const float* src_vs,
                            void* dst_k, void* dst_v, float* dst_ks, float* dst_vs, int64_t block_bytes,
                            int64_t scales_per_blk, const int64_t* pairs, int32_t P, int32_t src_NB,
                            int32_t dst_NB, hipStream_t st);
pa_status launch_quantize_and_cache(const void* key, const void* value, pa_dtype src_dtype, void* k_cache,
                                    void* v_cache, pa_dtype kv_dtype, float* k_scales, float* v_scales,
                                    int32_t scale_mode, float k_static, float v_static, const int64_t* slots,
                                    int32_t T, int32_t Hkv, int32_t D, int32_t BS, int32_t NB, hipStream_t st);

}  // namespace pa
