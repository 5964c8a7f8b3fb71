// Host side of libpa: status strings, per-thread error messages, argument
// validation and the decode plan (which kernel, how the context is split),
// then the launches.  No device memory is allocated here.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>

#include "pa_internal.h"

namespace pa {

static thread_local char g_last_error[512] = "";

pa_status fail(pa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static bool valid_dtype(int t) { return t == PA_F32 || t == PA_BF16 || t == PA_I8 || t == PA_FP8_E4M3; }
static bool valid_scale_mode(int m) { return m == PA_SCALE_BLOCK || m == PA_SCALE_TOKEN; }

// Waves a decode launch should put on the chip (256 CUs on MI355X).  The
// matrix-core kernel keeps two 16-token tiles in flight per wave: with a
// bf16 cache that is 16 KB, and about 2.5 waves per CU (~40 KB of loads in
// flight per CU) measured fastest on the 70B-shaped layer, while five per
// CU lost 10 %.  1-byte tiles carry half the bytes for the same arithmetic:
// on the same layer with int8 or E4M3 codes, 10 waves per CU (512-token
// partitions) measured 61-65 % of peak against 52-58 % at 5 per CU and
// 38-49 % at 2.5.  A bf16 cache at head_dim 64 also carries half the bytes
// per tile: on the 70B-shaped batch at head_dim 64, 1,280 waves (8
// partitions) read 71.8-72.3 % against 62.0-62.4 % with 640 (and 67-69 %
// with 12 or 16 partitions).  The vector-ALU kernel keeps one tile in
// flight; five waves per CU.
// SIMDs of the chip (256 compute units of 4)
constexpr int64_t kSimds = 1024;

static int target_waves(KernelKind kind, pa_dtype kv, int head_dim) {
  if (kind == KERNEL_MFMA) return quantised(kv) ? 2560 : head_dim == 64 ? 1280 : 640;
  return 1280;
}

// A ragged batch (mean length under 3/4 of the maximum) is cut into short
// partitions instead: about 20 waves per CU, which the dispatcher hands
// out as earlier ones finish, so the long sequences no longer set the
// kernel's end.  Measured on one-layer batches with log-normal and uniform
// lengths (int8 and bf16 caches): ~5,000 waves of <= 16 tiles beat both
// fewer longer waves and more shorter ones.
constexpr int64_t kRaggedWaves = 5120;
// Waves of a balanced split (one launch, all kv heads).  For 1-byte codes
// 1,920 read 0.7-2 points more than 2,560 on the int8, per-token int8 and
// E4M3 layers (64 log-normal sequences; int8 54.8-55.6 % of HBM peak against
// 54.0-54.9 %), and more than 1,280 and 2,240; 3,072 was within noise of it.
static int64_t balanced_waves(int32_t kv_dtype) { return kv_dtype == PA_BF16 ? 640 : 1920; }

// Waves for the items over a shared prefix.  Measured on the prefix-sharing
// layer (50 sequences, 1,984 shared tokens, 32/8 heads): 2 partitions of
// 62 tiles (~1,000 waves) beat 4 to 16 shorter ones, whose extra partials
// cost the merge more than the shorter chains save.
constexpr int64_t kPrefixWaves = 1024;
static bool is_ragged(const pa_decode_args* a, int64_t total) {
  return total * 4 < (int64_t)a->num_seqs * a->max_context_len * 3;
}

pa_status plan_decode(const pa_decode_args* a, DecodePlan* p) {
  if (!a) return fail(PA_ERR_INVALID, "pa_decode: args is NULL");
  if (a->struct_size != sizeof(pa_decode_args))
    return fail(PA_ERR_INVALID, "pa_decode: struct_size %zu, expected %zu (ABI mismatch)",
                a->struct_size, sizeof(pa_decode_args));
  if (a->num_seqs < 0) return fail(PA_ERR_INVALID, "pa_decode: num_seqs < 0");
  if (a->num_q_heads <= 0 || a->num_kv_heads <= 0 || a->head_dim <= 0 || a->block_size <= 0 ||
      a->num_blocks <= 0 || a->max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID, "pa_decode: head counts, head_dim, block_size, num_blocks and "
                                "max_blocks_per_seq must be positive");
  if (a->num_q_heads % a->num_kv_heads)
    return fail(PA_ERR_INVALID, "pa_decode: num_q_heads %d is not a multiple of num_kv_heads %d",
                a->num_q_heads, a->num_kv_heads);
  const int G = a->num_q_heads / a->num_kv_heads;
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(PA_ERR_INVALID, "pa_decode: head_dim %d not in {64, 128}", a->head_dim);
  if (a->block_size != 16 && a->block_size != 32)
    return fail(PA_ERR_INVALID, "pa_decode: block_size %d not in {16, 32}", a->block_size);
  if (!valid_dtype(a->q_dtype) || !valid_dtype(a->kv_dtype) || !valid_dtype(a->out_dtype))
    return fail(PA_ERR_INVALID, "pa_decode: unknown dtype code");
  if (a->out_dtype != PA_F32 && a->out_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: out_dtype must be PA_F32 or PA_BF16");
  if (quantised(a->q_dtype)) return fail(PA_ERR_UNSUPPORTED, "pa_decode: quantised queries");
  const bool i8 = quantised(a->kv_dtype);  // 1-byte codes with scales
  if (i8 != (a->k_scales != nullptr) || i8 != (a->v_scales != nullptr))
    return fail(PA_ERR_INVALID, "pa_decode: k_scales/v_scales must be given exactly for quantised caches");
  if (i8 && !valid_scale_mode(a->kv_scale_mode))
    return fail(PA_ERR_INVALID, "pa_decode: kv_scale_mode %d not a pa_scale_mode", a->kv_scale_mode);
  if (!std::isfinite(a->scale)) return fail(PA_ERR_INVALID, "pa_decode: scale is not finite");
  if ((a->new_key == nullptr) != (a->new_value == nullptr))
    return fail(PA_ERR_INVALID, "pa_decode: give both new_key and new_value, or neither");
  if (a->new_key && i8 && (a->kv_scale_mode != PA_SCALE_TOKEN || a->head_dim != 128))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: the fused write into a quantised cache needs per-token scales "
                                    "and head_dim 128 (else pa_quantize_and_cache first)");
  if (a->max_context_len < 0 || (int64_t)a->max_context_len > (int64_t)a->max_blocks_per_seq * a->block_size)
    return fail(PA_ERR_INVALID, "pa_decode: max_context_len %d outside [0, max_blocks_per_seq*block_size]",
                a->max_context_len);
  if (a->partition_tokens < 0 || a->partition_tokens % 16 || a->partition_tokens > kMaxPartitionBlocks * a->block_size)
    return fail(PA_ERR_INVALID, "pa_decode: partition_tokens %d is not a multiple of 16 in [0, %d*block_size]",
                a->partition_tokens, kMaxPartitionBlocks);
  if (a->kernel < 0 || a->kernel > 2) return fail(PA_ERR_INVALID, "pa_decode: kernel %d not in {0, 1, 2}", a->kernel);
  const bool mq = a->query_start_loc != nullptr;
  if (a->shared_prefix_len < 0 || (a->shared_prefix_len > 0 && !a->shared_prefix_table))
    return fail(PA_ERR_INVALID, "pa_decode: shared_prefix_len %d needs shared_prefix_table", a->shared_prefix_len);
  if (a->shared_prefix_len % a->block_size)
    return fail(PA_ERR_INVALID, "pa_decode: shared_prefix_len %d is not a multiple of block_size %d",
                a->shared_prefix_len, a->block_size);
  if (a->shared_prefix_len > a->max_context_len)
    return fail(PA_ERR_INVALID, "pa_decode: shared_prefix_len %d exceeds max_context_len %d", a->shared_prefix_len,
                a->max_context_len);
  if (mq && (a->num_queries < 0 || a->max_query_len < 1))
    return fail(PA_ERR_INVALID, "pa_decode: with query_start_loc, num_queries >= 0 and max_query_len >= 1");
  if (mq && a->new_key)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: no fused cache write with several query rows per sequence");
  const int64_t seq_tokens = (int64_t)(a->num_seqs > 0 ? a->num_seqs : 0) * a->max_context_len;
  if (a->total_context_len < 0 || a->total_context_len > seq_tokens)
    return fail(PA_ERR_INVALID, "pa_decode: total_context_len %lld outside [0, num_seqs * max_context_len]",
                (long long)a->total_context_len);

  // matrix-core kernel: bf16 queries with a bf16, int8 or E4M3 cache
  const bool mfma_ok = a->q_dtype == PA_BF16 && (a->kv_dtype == PA_BF16 || i8);
  if (mq && (!mfma_ok || a->kernel == KERNEL_VALU))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: several query rows per sequence need the matrix-core kernel "
                                    "(bf16 queries with a bf16, int8 or E4M3 cache)");
  KernelKind kind;
  if (a->new_key && i8 && (!mfma_ok || a->kernel == KERNEL_VALU))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: the fused write into a quantised cache needs the matrix-core "
                                    "kernel (bf16 queries)");
  if (a->kernel == KERNEL_MFMA) {
    if (!mfma_ok)
      return fail(PA_ERR_UNSUPPORTED, "pa_decode: matrix-core kernel needs bf16 queries with a bf16, int8 "
                                      "or E4M3 cache");
    kind = KERNEL_MFMA;
  } else if (a->kernel == KERNEL_VALU) {
    kind = KERNEL_VALU;
  } else {
    kind = mfma_ok ? KERNEL_MFMA : KERNEL_VALU;
  }

  p->kind = kind;
  p->G = G;
  int hpw = 1;
  while (hpw < G && hpw < 8) hpw *= 2;
  p->heads_per_wave = kind == KERNEL_VALU ? hpw : G;
  p->head_groups = kind == KERNEL_VALU ? (G + hpw - 1) / hpw : 1;
  // columns of the MFMA kernel: G heads x up to max_query_len rows (one
  // row without query_start_loc), 16 at a time; more than 16 query heads
  // per kv head take several column groups as several rows would
  const int64_t cg = ((int64_t)G * (mq ? a->max_query_len : 1) + 15) / 16;
  if (cg > 4096)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: %lld groups of 16 (query row, head) columns per kv head (max 4096)",
                (long long)cg);
  // (the vector-ALU kernel takes the heads in head groups instead)
  p->cgroups = kind == KERNEL_MFMA ? (int)cg : 1;
  p->ncg = p->cgroups >= 2 ? 2 : 1;
  p->cg_waves = (p->cgroups + p->ncg - 1) / p->ncg;
  p->rows = (int64_t)(mq ? a->num_queries : (a->num_seqs > 0 ? a->num_seqs : 0)) * a->num_q_heads;
  // Several query rows with more than one wave of column groups per item
  // (head_dim 128; bf16, int8 or E4M3 cache): the item's waves share each
  // K/V tile through LDS in workgroups (else each wave reads every tile
  // itself), one column group per wave in workgroups of kSharedWaves.  On
  // the 70B-shaped layer with a 64-row chunk per sequence (32 column groups
  // per item) the per-wave kernel is bound by those re-reads: 347-349
  // against 384-389 TFLOP/s at first (bf16; int8 375 against 442-449).
  p->shared_tiles = kind == KERNEL_MFMA && mq && a->head_dim == 128 && p->cg_waves >= 2;
  if (p->shared_tiles) {
    p->ncg = 1;
    p->cg_waves = p->cgroups;
  }

  const int64_t max_tiles = (int64_t)kMaxPartitionBlocks * a->block_size / 16;
  const int64_t total = a->total_context_len > 0 ? a->total_context_len : seq_tokens;
  const int64_t target = target_waves(kind, a->kv_dtype, a->head_dim);

  // Partition length for `seqs` sequences of at most max_len tokens (sum
  // total_len), each split over `per_seq` items per partition of `wpi`
  // waves each (the waves of an item share its tiles); `wave_mult` scales
  // the wave target (waves carrying two column groups), `tgt` replaces it.
  auto choose_split = [&](int64_t max_len, int64_t total_len, int64_t seqs, int64_t per_seq, int64_t wave_mult,
                          bool ragged_ok, int64_t wpi = 1, int64_t tgt = 0) -> int {
    const int64_t tiles = max_len > 0 ? (max_len + 15) / 16 : 1;
    if (ragged_ok && seqs > 0 && total_len * 4 < seqs * max_len * 3) {
      // Ragged lengths: about total/P + S/2 partitions per wave column;
      // choose P for ~kRaggedWaves waves, at least 4 tiles per wave, at
      // most kMaxPartitionBlocks blocks and kMaxRaggedPartitions partitions.
      int64_t room = kRaggedWaves - per_seq * wpi * seqs / 2;
      if (room < kRaggedWaves / 4) room = kRaggedWaves / 4;
      int64_t per = (per_seq * wpi * total_len + 16 * room - 1) / (16 * room);  // tiles per partition
      const int64_t min_per = (tiles + kMaxRaggedPartitions - 1) / kMaxRaggedPartitions;
      if (per < min_per) per = min_per;
      if (per < 4 * wpi) per = 4 * wpi;
      if (per > max_tiles) per = max_tiles;
      if (per > tiles) per = tiles;
      return (int)(16 * per);
    }
    // Near-equal lengths: nP equal partitions so the grid holds about
    // target waves, within [4 tiles per wave, kMaxPartitionBlocks blocks]
    // per partition and at most kMaxAutoPartitions partitions.
    const int64_t groups = (seqs > 0 ? seqs : 1) * per_seq * wpi;
    const int64_t tw = (tgt ? tgt : target) * wave_mult;
    // A wave carrying two column groups computes about twice as long per
    // tile, and two such waves on one SIMD slow each other: at most one
    // per SIMD.  The 70B-shaped layer with 4 query rows per sequence (160
    // items) read 70.6-71.5 % of HBM peak with 6 partitions (960 waves),
    // 65.7-66.8 % with 8 (1,280), 64 % with 7 and 67 % with 5.
    int64_t nP = (wave_mult == 2 && !tgt) ? kSimds / groups : (tw + groups / 2) / groups;
    if (nP < 1) nP = 1;
    if (nP > kMaxAutoPartitions) nP = kMaxAutoPartitions;
    if (nP > (tiles + 4 * wpi - 1) / (4 * wpi)) nP = (tiles + 4 * wpi - 1) / (4 * wpi);
    int64_t per = (tiles + nP - 1) / nP;
    if (per > max_tiles) per = max_tiles;
    return (int)(16 * per);
  };

  // Shared prefix (cascade): every sequence's first shared_prefix_len tokens
  // are the blocks of shared_prefix_table.  Prefix items attend all
  // sequences' queries to those blocks (K/V read once per 16 columns of
  // sequences x query heads), the other items each sequence to the rest of
  // its tokens, in one launch of kCascadeWaves-wave items; the merge
  // combines both.  Matrix-core kernel, one query row per sequence;
  // otherwise the hint is ignored.  The prefix's tiles are re-read by every
  // column group (mostly from cache), so its items are latency-bound, not
  // bandwidth-bound: they get kPrefixWaves waves.  The rest of each
  // sequence is split by the near-equal rule; with S x Hkv items of 4
  // waves above the wave target it stays one partition per sequence.
  p->cascade = false;
  p->prefix_partitions = 0;
  if (a->shared_prefix_len > 0 && kind == KERNEL_MFMA && !mq && p->cgroups == 1 && a->num_seqs > 0) {
    // A given partition_tokens sets both passes' partition length.
    p->cascade = true;
    const int64_t pcg = ((int64_t)G * a->num_seqs + 15) / 16;
    p->prefix_cgroups = (int)pcg;
    const int Pp = a->partition_tokens ? a->partition_tokens
                                       : choose_split(a->shared_prefix_len, a->shared_prefix_len, 1,
                                                      (int64_t)a->num_kv_heads * pcg, 1, false, kCascadeWaves,
                                                      kPrefixWaves);
    p->prefix_tokens = Pp;
    p->prefix_partitions = (a->shared_prefix_len + Pp - 1) / Pp;
    const int64_t rest_max = a->max_context_len - a->shared_prefix_len;
    const int64_t rest_total = total - (int64_t)a->num_seqs * a->shared_prefix_len;
    const int P = a->partition_tokens ? a->partition_tokens
                                      : choose_split(rest_max, rest_total > 0 ? rest_total : 0, a->num_seqs,
                                                     a->num_kv_heads, 1, false, kCascadeWaves);
    p->partition_tokens = P;
    p->num_partitions = rest_max > 0 ? (int)((rest_max + P - 1) / P) : 0;
  } else {
    int P = a->partition_tokens;
    if (P == 0)
      P = choose_split(a->max_context_len, total, a->num_seqs, (int64_t)a->num_kv_heads * p->head_groups *
                       p->cg_waves, p->ncg, !mq);
    p->partition_tokens = P;
    p->num_partitions = a->max_context_len > 0 ? (a->max_context_len + P - 1) / P : 1;
  }
  p->ws_partitions = p->prefix_partitions + p->num_partitions;
  // Balanced split for a skewed batch (length hint given, mean under 1/4 of
  // the maximum, matrix-core decode with the library's own split): every
  // wave gets an equal range of its head's tiles, whatever the lengths, so
  // long and short sequences cost no per-partition start-up or partial
  // beyond one per (range, sequence) piece.  Measured on log-normal
  // lengths (mean / max 0.12): bf16 59 -> 70 %, int8 44 -> 50 % of HBM
  // peak; on U[200, 2048] (mean / max 0.55) the short partitions of the
  // ragged rule stay ahead by ~1 point.
  p->balanced = false;
  if (kind == KERNEL_MFMA && !mq && p->cgroups == 1 && !p->cascade && a->partition_tokens == 0 && a->total_context_len > 0 &&
      a->num_seqs > 0 && a->num_seqs <= kBalancedWideMaxSeqs && a->max_context_len > 0 &&
      a->total_context_len * 4 < (int64_t)a->num_seqs * a->max_context_len) {
    const int64_t max_tiles = (a->max_context_len + 15) / 16;
    // tiles per head from the hint (an upper bound on the true count), and
    // enough waves that no wave needs a second range of at most
    // kBalancedMaxTiles (a second range doubles that wave's time)
    const int64_t t_hint = (a->total_context_len + 15) / 16 + a->num_seqs;
    int64_t wh = (balanced_waves(a->kv_dtype) + a->num_kv_heads - 1) / a->num_kv_heads;
    if (wh < (t_hint + kBalancedMaxTiles - 1) / kBalancedMaxTiles) wh = (t_hint + kBalancedMaxTiles - 1) / kBalancedMaxTiles;
    int64_t pw = (t_hint + wh - 1) / wh;
    if (pw < 1) pw = 1;
    if (pw > kBalancedMaxTiles) pw = kBalancedMaxTiles;
    // a sequence of n tiles meets at most floor((n - 1) / pw) + 2 ranges;
    // the kernel keeps ranges >= max_tiles / (slots - 1) tiles so that
    // every sequence's pieces fit its slots, whatever the true lengths
    const int64_t slots = (max_tiles + pw - 1) / pw + 1;
    p->balanced = true;
    p->balanced_waves = (int)wh;
    p->balanced_min_tiles = (int)((max_tiles + slots - 2) / (slots - 1));
    p->num_partitions = (int)slots;
    p->ws_partitions = (int)slots;
  }
  // Groups: with one column group per (sequence, kv head) (one query row,
  // or a few rows of few heads), at most kMaxGroupWaves partitions and at
  // least kGroupMinItems (sequence, kv head) items, the partitions of an
  // item are the waves of one workgroup and combine through LDS, so the
  // call needs neither partials nor the merge launch.  A workgroup runs on
  // one compute unit, so with fewer items than units the grouped launch
  // leaves units idle: on the 70B-shaped layer (160 items of 4
  // partitions) it read 79.3 % of HBM peak against 79.9 % with partials
  // and the merge; on the 13B-shaped one (1,280 items) 75.3 % against
  // 70.6 %.  An automatic split is re-cut into exactly as many partitions
  // as the group has waves.  An automatic split of a short batch (longest
  // sequence at most kGroupShortTiles tiles) into more partitions than a
  // workgroup takes -- the ragged rule's short partitions -- is re-cut into
  // 4-wave groups instead: on 32 to 64 sequences of 50 to 1,000 or 2,000
  // tokens (8 kv heads, bf16 or int8) that took 0.66 to 0.87 of the time of
  // the short partitions, their partials and the merge, and 0.87 to 1.12 of
  // 8-wave groups.  A small batch (at most kGroupSmallTiles tiles over all
  // its (sequence, kv head) items) takes at most 4 waves per group: on 32 to
  // 100 sequences of 50..500 tokens (8 kv heads) 4-wave groups took 0.85 to
  // 0.93 of the time of 8-wave ones for bf16, 0.90 to 1.02 for int8; on 128
  // sequences of 50..1,000 tokens (33,600 tiles) and the 13B-shaped layer
  // 8 waves stay ahead.
  p->grouped = false;
  p->group_waves = 1;
  const int64_t ctx_tiles = ((int64_t)a->max_context_len + 15) / 16;
  const bool short_recut = a->partition_tokens == 0 && p->num_partitions > kMaxGroupWaves &&
                           ctx_tiles <= kGroupShortTiles;
  if (kind == KERNEL_MFMA && p->cgroups == 1 && !p->cascade && !p->balanced && p->num_partitions >= 2 &&
      (p->num_partitions <= kMaxGroupWaves || short_recut) &&
      (int64_t)a->num_seqs * a->num_kv_heads >= kGroupMinItems) {
    int w = 2;
    while (w < p->num_partitions && w < kMaxGroupWaves) w *= 2;
    const int64_t all_tiles = (total / 16 + a->num_seqs) * a->num_kv_heads;
    if (short_recut || (a->partition_tokens == 0 && w > 4 && all_tiles <= kGroupSmallTiles)) w = 4;
    if (a->partition_tokens == 0) {
      const int64_t tiles = ctx_tiles;
      p->partition_tokens = (int)(16 * ((tiles + w - 1) / w));
      p->num_partitions = (int)((a->max_context_len + p->partition_tokens - 1) / p->partition_tokens);
    }
    p->grouped = true;
    p->group_waves = w;
    p->ws_partitions = 1;
  }
  p->workspace_bytes = workspace_layout(a, *p).bytes;
  return PA_OK;
}

}  // namespace pa

using namespace pa;

extern "C" {

const char* pa_status_string(pa_status s) {
  // A C caller may pass any int; read it as one (an enum value outside the
  // enumerators' range is undefined in C++).
  static_assert(sizeof(pa_status) == sizeof(int), "pa_status is an int");
  int code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID: return "PA_ERR_INVALID";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_OOM: return "PA_ERR_OOM";
    case PA_ERR_STATE: return "PA_ERR_STATE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
  }
  return "PA_ERR_UNKNOWN";
}

const char* pa_last_error(void) { return g_last_error; }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

pa_status pa_decode_workspace_size(const pa_decode_args* a, size_t* bytes) {
  DecodePlan p;
  if (!bytes) return fail(PA_ERR_INVALID, "pa_decode_workspace_size: bytes is NULL");
  pa_status s = plan_decode(a, &p);
  if (s != PA_OK) return s;
  *bytes = p.workspace_bytes;
  return PA_OK;
}

size_t pa_decode_workspace_bytes(const pa_decode_args* a) {
  DecodePlan p;
  return plan_decode(a, &p) == PA_OK ? p.workspace_bytes : SIZE_MAX;
}

pa_status pa_decode(const pa_decode_args* a) {
  DecodePlan p;
  pa_status s = plan_decode(a, &p);
  if (s != PA_OK) return s;
  if (a->num_seqs == 0) return PA_OK;
  if (!a->out || !a->q || !a->k_cache || !a->v_cache || !a->block_tables || !a->context_lens)
    return fail(PA_ERR_INVALID, "pa_decode: a required device pointer is NULL");
  if (a->query_start_loc && !aligned(a->query_start_loc, 4))
    return fail(PA_ERR_INVALID, "pa_decode: query_start_loc must be 4-byte aligned");
  if (a->shared_prefix_len > 0 && !aligned(a->shared_prefix_table, 4))
    return fail(PA_ERR_INVALID, "pa_decode: shared_prefix_table must be 4-byte aligned");
  if (!aligned(a->out, 16) || !aligned(a->q, 16) || !aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) ||
      !aligned(a->new_key, 16) || !aligned(a->new_value, 16))
    return fail(PA_ERR_INVALID, "pa_decode: out, q, the caches and new_key/new_value must be 16-byte aligned");
  const size_t sa = a->kv_scale_mode == PA_SCALE_TOKEN ? 16 : 4;
  if (!aligned(a->block_tables, 4) || !aligned(a->context_lens, 4) ||
      (a->k_scales && (!aligned(a->k_scales, sa) || !aligned(a->v_scales, sa))))
    return fail(PA_ERR_INVALID, "pa_decode: tables and lengths must be 4-byte aligned, scales 4-byte "
                                "(per block) or 16-byte (per token) aligned");
  if (p.workspace_bytes) {
    if (!a->workspace || a->workspace_bytes < p.workspace_bytes)
      return fail(PA_ERR_INVALID, "pa_decode: workspace of %zu bytes needed, %zu given", p.workspace_bytes,
                  a->workspace ? a->workspace_bytes : (size_t)0);
    if (!aligned(a->workspace, 16)) return fail(PA_ERR_INVALID, "pa_decode: workspace must be 16-byte aligned");
  }
  hipStream_t st = (hipStream_t)a->stream;
  if (debug_enabled() && (s = debug_check_decode(a, st)) != PA_OK) return s;
  // a bf16 output: the kernels write the fp32 rows into the workspace, and
  // one more pass rounds them into out
  pa_decode_args f = *a;
  if (a->out_dtype == PA_BF16) {
    f.out = (char*)a->workspace + workspace_layout(a, p).out_offset;
    f.out_dtype = PA_F32;
  }
  s = p.kind == KERNEL_MFMA ? launch_decode_mfma(&f, p, st) : launch_decode_valu(&f, p, st);
  if (s == PA_OK && p.ws_partitions > 1) s = launch_decode_merge(&f, p, st);
  if (s == PA_OK && a->out_dtype == PA_BF16)
    s = launch_f32_to_bf16((const float*)f.out, a->out, (size_t)p.rows * a->head_dim, st);
  return s;
}

pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                          const int32_t* seq_idx, const int32_t* positions, const int32_t* context_lens,
                          int32_t num_tokens, int32_t block_size, int64_t* slot_mapping, void* stream) {
  if (num_tokens < 0 || num_seqs < 0) return fail(PA_ERR_INVALID, "pa_slot_mapping: negative count");
  if (max_blocks_per_seq <= 0 || block_size <= 0)
    return fail(PA_ERR_INVALID, "pa_slot_mapping: max_blocks_per_seq and block_size must be positive");
  if ((positions == nullptr) == (context_lens == nullptr))
    return fail(PA_ERR_INVALID, "pa_slot_mapping: give exactly one of positions and context_lens");
  if (!seq_idx && num_tokens > num_seqs)
    return fail(PA_ERR_INVALID, "pa_slot_mapping: without seq_idx, num_tokens (%d) must not exceed num_seqs (%d)",
                num_tokens, num_seqs);
  if (num_tokens == 0) return PA_OK;
  if (!block_tables || !slot_mapping) return fail(PA_ERR_INVALID, "pa_slot_mapping: NULL device pointer");
  return launch_slot_mapping(block_tables, max_blocks_per_seq, num_seqs, seq_idx, positions, context_lens, num_tokens,
                             block_size, slot_mapping, (hipStream_t)stream);
}

static pa_status check_cache_shape(const char* fn, pa_dtype kv, int32_t Hkv, int32_t D, int32_t BS, int32_t NB) {
  if (!valid_dtype(kv)) return fail(PA_ERR_INVALID, "%s: unknown dtype code", fn);
  if (Hkv <= 0 || NB <= 0) return fail(PA_ERR_INVALID, "%s: num_kv_heads and num_blocks must be positive", fn);
  if (D != 64 && D != 128) return fail(PA_ERR_INVALID, "%s: head_dim %d not in {64, 128}", fn, D);
  if (BS != 16 && BS != 32) return fail(PA_ERR_INVALID, "%s: block_size %d not in {16, 32}", fn, BS);
  return PA_OK;
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache, pa_dtype kv_dtype,
                               const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t num_blocks, void* stream) {
  pa_status s = check_cache_shape("pa_reshape_and_cache", kv_dtype, num_kv_heads, head_dim, block_size, num_blocks);
  if (s != PA_OK) return s;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_reshape_and_cache: num_tokens < 0");
  if (quantised(kv_dtype))
    return fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: quantised caches are written by pa_quantize_and_cache");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID, "pa_reshape_and_cache: NULL device pointer");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID, "pa_reshape_and_cache: key, value and caches must be 16-byte aligned");
  if (debug_enabled() && (s = debug_check_slots(slot_mapping, num_tokens, num_blocks, block_size, (hipStream_t)stream,
                                                "pa_reshape_and_cache")) != PA_OK)
    return s;
  return launch_reshape_and_cache(key, value, k_cache, v_cache, dtype_bytes(kv_dtype), slot_mapping, num_tokens,
                                  num_kv_heads, head_dim, block_size, num_blocks, (hipStream_t)stream);
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, pa_dtype kv_dtype, float* k_scales, float* v_scales,
                         int32_t scale_mode, const int64_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, void* stream) {
  pa_status s = check_cache_shape("pa_copy_blocks", kv_dtype, num_kv_heads, head_dim, block_size, num_blocks);
  if (s != PA_OK) return s;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "pa_copy_blocks: num_pairs < 0");
  const bool q8 = quantised(kv_dtype);
  if (q8 != (k_scales != nullptr) || q8 != (v_scales != nullptr))
    return fail(PA_ERR_INVALID, "pa_copy_blocks: k_scales/v_scales must be given exactly for quantised caches");
  if (q8 && !valid_scale_mode(scale_mode))
    return fail(PA_ERR_INVALID, "pa_copy_blocks: scale_mode %d not a pa_scale_mode", scale_mode);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return fail(PA_ERR_INVALID, "pa_copy_blocks: NULL device pointer");
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 8))
    return fail(PA_ERR_INVALID, "pa_copy_blocks: caches must be 16-byte aligned");
  if (debug_enabled() && (s = debug_check_pairs(block_pairs, num_pairs, num_blocks, num_blocks, true,
                                                (hipStream_t)stream, "pa_copy_blocks")) != PA_OK)
    return s;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * dtype_bytes(kv_dtype);
  return launch_block_copy(k_cache, v_cache, k_scales, v_scales, k_cache, v_cache, k_scales, v_scales, block_bytes,
                           q8 ? scales_per_block(scale_mode, num_kv_heads, block_size) : 0, block_pairs, num_pairs,
                           num_blocks, num_blocks, (hipStream_t)stream);
}

// Address under which a kernel reaches p: device memory as is, pinned host
// memory (hipHostMalloc) through its device mapping; NULL for anything else
// (pageable host memory would fault the GPU, so it is refused).
static const void* device_view(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged || at.type == hipMemoryTypeUnified)
    return p;
  if (at.type == hipMemoryTypeHost) return at.devicePointer;
  return nullptr;
}

pa_status pa_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scales, const float* src_v_scales,
                         void* dst_k, void* dst_v, float* dst_k_scales, float* dst_v_scales, pa_dtype kv_dtype,
                         int32_t scale_mode, const int64_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t src_num_blocks, int32_t dst_num_blocks,
                         void* stream) {
  pa_status s = check_cache_shape("pa_swap_blocks", kv_dtype, num_kv_heads, head_dim, block_size,
                                  src_num_blocks < dst_num_blocks ? src_num_blocks : dst_num_blocks);
  if (s != PA_OK) return s;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "pa_swap_blocks: num_pairs < 0");
  const int given = (src_k_scales != nullptr) + (src_v_scales != nullptr) + (dst_k_scales != nullptr) +
                    (dst_v_scales != nullptr);
  if (given != 0 && given != 4)
    return fail(PA_ERR_INVALID, "pa_swap_blocks: give all four scale arrays or none");
  if (given && !quantised(kv_dtype))
    return fail(PA_ERR_INVALID, "pa_swap_blocks: scales given for a cache that is not quantised");
  if (given && !valid_scale_mode(scale_mode))
    return fail(PA_ERR_INVALID, "pa_swap_blocks: scale_mode %d not a pa_scale_mode", scale_mode);
  if (num_pairs == 0) return PA_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_pairs)
    return fail(PA_ERR_INVALID, "pa_swap_blocks: NULL pointer");
  if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) || !aligned(dst_v, 16) ||
      !aligned(block_pairs, 8))
    return fail(PA_ERR_INVALID, "pa_swap_blocks: pools must be 16-byte aligned");
  const void* dv[9] = {src_k, src_v, dst_k, dst_v, block_pairs, src_k_scales, src_v_scales, dst_k_scales,
                       dst_v_scales};
  for (int i = 0; i < (given ? 9 : 5); ++i) {
    const void* v = device_view(dv[i]);
    if (!v) return fail(PA_ERR_INVALID, "pa_swap_blocks: argument %d is neither device nor pinned host memory", i);
    dv[i] = v;
  }
  if (debug_enabled() && (s = debug_check_pairs(block_pairs, num_pairs, src_num_blocks, dst_num_blocks,
                                                src_k == dst_k, (hipStream_t)stream, "pa_swap_blocks")) != PA_OK)
    return s;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * dtype_bytes(kv_dtype);
  return launch_block_copy(dv[0], dv[1], (const float*)dv[5], (const float*)dv[6], (void*)dv[2], (void*)dv[3],
                           (float*)dv[7], (float*)dv[8], block_bytes,
                           given ? scales_per_block(scale_mode, num_kv_heads, block_size) : 0,
                           (const int64_t*)dv[4], num_pairs, src_num_blocks, dst_num_blocks, (hipStream_t)stream);
}

pa_status pa_quantize_and_cache(const void* key, const void* value, pa_dtype src_dtype, void* k_cache, void* v_cache,
                                pa_dtype kv_dtype, float* k_scales, float* v_scales, int32_t scale_mode,
                                float k_static_scale, float v_static_scale, const int64_t* slot_mapping,
                                int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                int32_t num_blocks, void* stream) {
  pa_status s = check_cache_shape("pa_quantize_and_cache", kv_dtype, num_kv_heads, head_dim, block_size, num_blocks);
  if (s != PA_OK) return s;
  if (!quantised(kv_dtype))
    return fail(PA_ERR_INVALID, "pa_quantize_and_cache: kv_dtype must be PA_I8 or PA_FP8_E4M3");
  if (src_dtype != PA_F32 && src_dtype != PA_BF16)
    return fail(PA_ERR_INVALID, "pa_quantize_and_cache: src_dtype must be PA_F32 or PA_BF16");
  if (!valid_scale_mode(scale_mode))
    return fail(PA_ERR_INVALID, "pa_quantize_and_cache: scale_mode %d not a pa_scale_mode", scale_mode);
  if (scale_mode == PA_SCALE_BLOCK &&
      !(k_static_scale > 0.f && v_static_scale > 0.f && std::isfinite(k_static_scale) &&
        std::isfinite(v_static_scale)))
    return fail(PA_ERR_INVALID, "pa_quantize_and_cache: static scales must be positive and finite");
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_quantize_and_cache: num_tokens < 0");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !k_scales || !v_scales || !slot_mapping)
    return fail(PA_ERR_INVALID, "pa_quantize_and_cache: NULL device pointer");
  if (!aligned(key, 16) || !aligned(value, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(k_scales, 4) || !aligned(v_scales, 4) || !aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID, "pa_quantize_and_cache: key, value and caches must be 16-byte aligned");
  if (debug_enabled() && (s = debug_check_slots(slot_mapping, num_tokens, num_blocks, block_size, (hipStream_t)stream,
                                                "pa_quantize_and_cache")) != PA_OK)
    return s;
  return launch_quantize_and_cache(key, value, src_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales, scale_mode,
                                   k_static_scale, v_static_scale, slot_mapping, num_tokens, num_kv_heads, head_dim,
                                   block_size, num_blocks, (hipStream_t)stream);
}

}  // extern "C"
