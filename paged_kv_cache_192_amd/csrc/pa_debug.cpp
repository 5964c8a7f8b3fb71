// Debug checks of the device-side preconditions that pa.h leaves to the
// caller, enabled by the environment variable PA_DEBUG (any value but "" or
// "0"; read on every call).  The kernels themselves only guard memory
// safety: an out-of-range block id contributes nothing, a bad slot or pair
// is skipped.  These checks turn such inputs, and the ones that would give
// an order-dependent or silently partial result (duplicate slots,
// overlapping copies, a length above max_context_len), into PA_ERR_INVALID
// before anything is launched.
//
// The library allocates no device memory, so the index arrays (tables,
// lengths, row offsets, slots, pairs) are copied to the host on the
// caller's stream, which is then synchronised: under PA_DEBUG every checked
// call waits for the stream's earlier work.  While the stream is being
// captured into a graph nothing can be synchronised, and the checks are
// skipped.
#include <cstdlib>
#include <unordered_set>
#include <vector>

#include "pa_internal.h"

namespace pa {

bool debug_enabled() {
  const char* e = std::getenv("PA_DEBUG");
  return e && e[0] && !(e[0] == '0' && e[1] == '\0');
}

namespace {

// true when the stream is being captured (the checks are then skipped)
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

template <typename T>
pa_status fetch(const T* src, size_t n, std::vector<T>& out, hipStream_t st, const char* fn) {
  out.resize(n);
  if (n == 0) return PA_OK;
  hipError_t e = hipMemcpyAsync(out.data(), src, n * sizeof(T), hipMemcpyDefault, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PA_ERR_HIP, "%s (PA_DEBUG): copying an index array to the host: %s", fn, hipGetErrorString(e));
  }
  return PA_OK;
}

// Slots of a cache write: each non-negative one below num_slots and none
// repeated (negative slots are skipped by the write).
pa_status check_slots(const int64_t* slot_mapping, int32_t num_tokens, int64_t num_slots, hipStream_t st,
                      const char* fn) {
  std::vector<int64_t> slots;
  pa_status s = fetch(slot_mapping, (size_t)num_tokens, slots, st, fn);
  if (s != PA_OK) return s;
  std::unordered_set<int64_t> seen;
  for (int32_t t = 0; t < num_tokens; ++t) {
    const int64_t v = slots[t];
    if (v < 0) continue;
    if (v >= num_slots)
      return fail(PA_ERR_INVALID, "%s (PA_DEBUG): slot_mapping[%d] = %lld is not below num_blocks * block_size = %lld",
                  fn, t, (long long)v, (long long)num_slots);
    if (!seen.insert(v).second)
      return fail(PA_ERR_INVALID, "%s (PA_DEBUG): slot %lld appears twice in slot_mapping (at token %d)", fn,
                  (long long)v, t);
  }
  return PA_OK;
}

}  // namespace

pa_status debug_check_decode(const pa_decode_args* a, hipStream_t st) {
  const char* fn = "pa_decode";
  if (capturing(st) || a->num_seqs == 0) return PA_OK;
  const int32_t S = a->num_seqs, MB = a->max_blocks_per_seq, BS = a->block_size, NB = a->num_blocks;
  std::vector<int32_t> lens, tables;
  pa_status s = fetch(a->context_lens, (size_t)S, lens, st, fn);
  if (s == PA_OK) s = fetch(a->block_tables, (size_t)S * MB, tables, st, fn);
  if (s != PA_OK) return s;
  const int64_t row_cap = (int64_t)MB * BS;
  for (int32_t i = 0; i < S; ++i) {
    const int32_t n = lens[i];
    if (n < 0 || n > row_cap || n > a->max_context_len)
      return fail(PA_ERR_INVALID,
                  "%s (PA_DEBUG): context_lens[%d] = %d outside [0, %lld] (max_context_len %d, table row of %d "
                  "blocks)",
                  fn, i, n, (long long)(row_cap < a->max_context_len ? row_cap : a->max_context_len),
                  a->max_context_len, MB);
    const int32_t used = (n + BS - 1) / BS;
    for (int32_t b = 0; b < used; ++b) {
      const int32_t id = tables[(size_t)i * MB + b];
      if (id < 0 || id >= NB)
        return fail(PA_ERR_INVALID, "%s (PA_DEBUG): block_tables[%d][%d] = %d, not a block of the pool [0, %d)", fn,
                    i, b, id, NB);
    }
  }
  if (a->query_start_loc) {
    std::vector<int32_t> qsl;
    s = fetch(a->query_start_loc, (size_t)S + 1, qsl, st, fn);
    if (s != PA_OK) return s;
    if (qsl[0] != 0 || qsl[S] != a->num_queries)
      return fail(PA_ERR_INVALID, "%s (PA_DEBUG): query_start_loc runs from %d to %d, not from 0 to num_queries = %d",
                  fn, qsl[0], qsl[S], a->num_queries);
    for (int32_t i = 0; i < S; ++i) {
      const int32_t L = qsl[i + 1] - qsl[i];
      if (L < 0 || L > a->max_query_len || L > lens[i])
        return fail(PA_ERR_INVALID,
                    "%s (PA_DEBUG): sequence %d has %d query rows (max_query_len %d, context length %d)", fn, i, L,
                    a->max_query_len, lens[i]);
    }
  }
  const int32_t pb = a->shared_prefix_len > 0 ? a->shared_prefix_len / BS : 0;
  if (pb > 0) {
    std::vector<int32_t> prefix;
    s = fetch(a->shared_prefix_table, (size_t)pb, prefix, st, fn);
    if (s != PA_OK) return s;
    for (int32_t b = 0; b < pb; ++b)
      if (prefix[b] < 0 || prefix[b] >= NB)
        return fail(PA_ERR_INVALID, "%s (PA_DEBUG): shared_prefix_table[%d] = %d, not a block of the pool [0, %d)",
                    fn, b, prefix[b], NB);
    for (int32_t i = 0; i < S; ++i) {
      const int32_t used = (lens[i] + BS - 1) / BS;
      for (int32_t b = 0; b < pb && b < used && b < MB; ++b)
        if (tables[(size_t)i * MB + b] != prefix[b])
          return fail(PA_ERR_INVALID,
                      "%s (PA_DEBUG): block_tables[%d][%d] = %d but the shared prefix has block %d there", fn, i, b,
                      tables[(size_t)i * MB + b], prefix[b]);
    }
  }
  if (a->new_key) {
    // the fused write's slots (newest token of every sequence that has one
    // outside the shared prefix) must be distinct
    std::unordered_set<int64_t> seen;
    for (int32_t i = 0; i < S; ++i) {
      const int32_t n = lens[i];
      if (n < 1 || (pb > 0 && n <= a->shared_prefix_len)) continue;
      const int64_t slot = (int64_t)tables[(size_t)i * MB + (n - 1) / BS] * BS + (n - 1) % BS;
      if (!seen.insert(slot).second)
        return fail(PA_ERR_INVALID,
                    "%s (PA_DEBUG): the newest tokens of two sequences map to the same slot %lld (sequence %d)", fn,
                    (long long)slot, i);
    }
  }
  return PA_OK;
}

pa_status debug_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                            hipStream_t st, const char* fn) {
  if (capturing(st) || num_tokens == 0) return PA_OK;
  return check_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size, st, fn);
}

pa_status debug_check_pairs(const int64_t* block_pairs, int32_t num_pairs, int32_t src_num_blocks,
                            int32_t dst_num_blocks, bool same_pool, hipStream_t st, const char* fn) {
  if (capturing(st) || num_pairs == 0) return PA_OK;
  std::vector<int64_t> pairs;
  pa_status s = fetch(block_pairs, (size_t)num_pairs * 2, pairs, st, fn);
  if (s != PA_OK) return s;
  std::unordered_set<int64_t> dsts, srcs;
  for (int32_t p = 0; p < num_pairs; ++p) {
    const int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    const bool in_range = src >= 0 && src < src_num_blocks && dst >= 0 && dst < dst_num_blocks;
    if (same_pool && !in_range)
      return fail(PA_ERR_INVALID, "%s (PA_DEBUG): pair %d = (%lld, %lld) names a block outside [0, %d)", fn, p,
                  (long long)src, (long long)dst, src_num_blocks);
    if (!in_range) continue;  // skipped by the copy, as documented
    if (!dsts.insert(dst).second)
      return fail(PA_ERR_INVALID, "%s (PA_DEBUG): destination block %lld appears twice (pair %d)", fn,
                  (long long)dst, p);
    srcs.insert(src);
  }
  if (same_pool)
    for (int32_t p = 0; p < num_pairs; ++p)
      if (srcs.count(pairs[2 * p + 1]))
        return fail(PA_ERR_INVALID, "%s (PA_DEBUG): block %lld is both a source and a destination (pair %d)", fn,
                    (long long)pairs[2 * p + 1], p);
  return PA_OK;
}

}  // namespace pa
