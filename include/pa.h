/*
 * pa.h -- C ABI of libpa: paged-KV-cache decode attention for AMD MI355X
 * (gfx950), its companion cache writes and the block pool.
 *
 * The method (from French web pages on the KV cache and PagedAttention):
 *  - The KV cache keeps the key and value vectors of every processed token;
 *    they never change once written, and each decode step adds one token
 *    per request ("Cache KV en production", opening section and section
 *    "Un cache par requête, une mémoire commune").
 *  - The cache is cut into fixed-size physical blocks of 16 or 32 tokens; a
 *    per-sequence block table maps logical block i to a physical block
 *    anywhere in device memory (ia-vox KV-cache article, section
 *    "PagedAttention : la révolution de l'allocation mémoire"; glossary
 *    "PagedAttention & Gestion du KV-Cache", section 2 figure).
 *  - Decode attends with the newest token's query only (deeplearn.tn
 *    article, section "La taille réelle du cache KV").
 *  - Blocks are taken from a shared pool as a request grows and returned
 *    when it ends or is cancelled; shared prefixes point at the same
 *    blocks and are copied on write (glossary sections 3 and 4;
 *    "Cache KV en production", sections on paging and prefix caching).
 *
 * Conventions for every call:
 *  - Device pointers are HIP device memory owned by the caller; the
 *    library never allocates or frees device memory.  Host pointers are
 *    marked "host".
 *  - Device calls are asynchronous on `stream` (a hipStream_t; NULL is the
 *    null stream).  No call synchronises the host.  Faults inside a kernel
 *    surface at the caller's next synchronisation.
 *  - Argument errors visible on the host return PA_ERR_INVALID before any
 *    launch; unsupported combinations return PA_ERR_UNSUPPORTED; a failed
 *    launch returns PA_ERR_HIP.  pa_last_error() then holds a message for
 *    the calling thread.  Nothing is thrown across the ABI.
 *  - Contents of device arrays (table entries, slot ids, pair ids) are the
 *    caller's responsibility; the kernels skip or clamp nothing beyond what
 *    each call documents.
 *  - With the environment variable PA_DEBUG set (to anything but "" or
 *    "0"; read on every call), the calls check those contents before any
 *    launch and return PA_ERR_INVALID naming the first violation: decode
 *    table entries in use inside [0, num_blocks), context lengths within
 *    [0, min(max_context_len, max_blocks_per_seq * block_size)], query row
 *    offsets (from 0 to num_queries, at most max_query_len and the
 *    sequence's length each), table rows starting with the shared prefix,
 *    distinct slots for the fused write; cache-write slots inside the pool
 *    and distinct; copy pairs inside the pool with distinct destinations
 *    disjoint from the sources; distinct swap destinations.  The arrays are
 *    copied to the host on the call's stream, which is synchronised, so a
 *    checked call waits for the stream's earlier work; while the stream is
 *    being captured into a graph the checks are skipped.
 *  - Kernels are stateless and re-entrant; a pa_pool is not thread-safe.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = 1,     /* bad argument, detected on the host */
  PA_ERR_UNSUPPORTED = 2, /* valid but not implemented (dtype or shape) */
  PA_ERR_OOM = 3,         /* pool has fewer free blocks than asked */
  PA_ERR_STATE = 4,       /* pool: free or share of a block not held */
  PA_ERR_HIP = 5          /* a HIP runtime call failed */
} pa_status;

/* Element types.  PA_FP8_E4M3 is the OCP 8-bit floating-point E4M3 format
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN =
 * all ones, largest finite value 448).  PA_I8 and PA_FP8_E4M3 caches are
 * quantised: every stored code is multiplied by an fp32 scale. */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_I8 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Layout of the fp32 scales of a quantised cache (ia-vox KV-cache article,
 * section "Quantization du KV cache": a fixed scale per layer is the static
 * form, a scale recomputed for every token the dynamic form):
 *   PA_SCALE_BLOCK: one scale per (block, kv head), [num_blocks][num_kv_heads];
 *   PA_SCALE_TOKEN: one scale per (block, kv head, slot), i.e. per token,
 *                   [num_blocks][num_kv_heads][block_size]. */
typedef enum { PA_SCALE_BLOCK = 0, PA_SCALE_TOKEN = 1 } pa_scale_mode;

/* Static string naming a status code. */
const char* pa_status_string(pa_status s);
/* Message of the last failure on the calling thread ("" if none). */
const char* pa_last_error(void);
/* ABI version of this header (incremented on any incompatible change). */
#define PA_ABI_VERSION 6
int32_t pa_abi_version(void);

/* ------------------------------------------------------------------------
 * Decode attention
 * ------------------------------------------------------------------------
 * For every sequence s and query head h, with G = num_q_heads /
 * num_kv_heads, kv head g = h / G and n = context_lens[s]:
 *
 *   K_s[t] = k_cache[block_tables[s][t / BS]][g][t % BS][:]   (same for V)
 *   x_t    = scale * <q[s][h][:], K_s[t]>                      t = 0 .. n-1
 *   out[s][h][:] = sum_t softmax(x)_t * V_s[t]
 *
 * The query of the newest token attends over all n tokens of its
 * sequence, the newest included (write it first with
 * pa_reshape_and_cache).  n = 0 gives a row of zeros.  For quantised
 * caches (PA_I8, PA_FP8_E4M3) the stored code's value is multiplied by its
 * fp32 scale, K = k_scale * code and V = v_scale * code, the scale taken
 * per (block, kv head) or per token as kv_scale_mode says (see
 * pa_scale_mode).
 *
 * Layouts (row-major, densely packed):
 *   q             [num_seqs][num_q_heads][head_dim]          q_dtype
 *   k/v_cache     [num_blocks][num_kv_heads][block_size][head_dim]  kv_dtype
 *   k/v_scales    fp32, quantised caches only: [num_blocks][num_kv_heads]
 *                 (PA_SCALE_BLOCK) or [num_blocks][num_kv_heads][block_size]
 *                 (PA_SCALE_TOKEN)
 *   block_tables  [num_seqs][max_blocks_per_seq] int32; entries past
 *                 ceil(n / BS) are never used, but the matrix-core kernel
 *                 may load any entry of the row (in bounds of the row), so
 *                 every row must be allocated in full
 *   context_lens  [num_seqs] int32, 0 <= n <= max_blocks_per_seq * BS and
 *                 n <= max_context_len
 *   out           [num_seqs][num_q_heads][head_dim] fp32, or bf16
 * Slots at or beyond n inside a sequence's last block, and blocks no table
 * names, are never read: they (and their scales) may hold anything, NaN
 * included.
 *
 * Supported: head_dim in {64, 128}; block_size in {16, 32};
 * q_dtype in {PA_F32, PA_BF16}; kv_dtype in {PA_F32, PA_BF16, PA_I8,
 * PA_FP8_E4M3};
 * out_dtype PA_F32 or PA_BF16 (the fp32 result rounded to nearest even
 * by one more pass over it, which takes num_seqs * num_q_heads * head_dim
 * fp32 of workspace; fp32 is the direct form); num_q_heads a multiple of
 * num_kv_heads (any number of
 * query heads per kv head: the matrix-core kernel takes them 16 at a time,
 * two groups of 16 per wave).  All of q, caches and out 16-byte aligned.
 *
 * Long contexts are split into partitions of `partition_tokens` tokens
 * (0 = chosen by the library), each computed by its own wave and merged by
 * a second kernel in partition order.  The library's choice uses
 * max_context_len and, when given, `total_context_len` (the sum of
 * context_lens over the batch, known to the caller that built the tables):
 * a batch whose lengths are close to the maximum is cut into a few long
 * partitions per sequence; a ragged one into many short ones, so that no
 * wave is left with a long sequence at the end.  The hint shapes only the
 * split (and so the workspace size), never the result; 0 means unknown
 * (every sequence taken at max_context_len).  With at most 8 partitions,
 * at least 256 (sequence, kv head) pairs and one group of 16 (query row,
 * head) columns per pair on the matrix-core kernel, a pair's partitions
 * run as the waves of one workgroup and are combined there (no merge
 * kernel, no workspace; the library's own split is then re-cut into 2, 4
 * or 8 equal partitions).  Otherwise the merge needs `workspace` of at
 * least the size pa_decode_workspace_size reports for the same arguments
 * (NULL is fine when that size is 0).  The workspace is scratch of the
 * call: its contents are not needed before or after it.  Calls that may
 * run concurrently need separate workspaces.
 *
 * Optional fused cache write: when `new_key` and `new_value` are given
 * ([num_seqs][num_kv_heads][head_dim] of kv_dtype, device), the call first
 * stores, for every sequence with n >= 1, the newest token's key and value
 * into the slot of position n - 1 (block_tables[s][(n-1)/BS], slot
 * (n-1) % BS, every kv head) and attends with them.  The result, cache
 * bytes included, is that of pa_slot_mapping (context_lens form) +
 * pa_reshape_and_cache + pa_decode, in one launch.  n must not exceed
 * max_context_len.  For a quantised cache with per-token scales
 * (PA_SCALE_TOKEN) at head_dim 128 on the matrix-core kernel, new_key and
 * new_value are bf16 rows: the call quantises them exactly as
 * pa_quantize_and_cache with dynamic scales would, stores the codes and
 * the two scales (k_scales and v_scales are then written, despite their
 * const type) and attends with them; the result, cache and scale bytes
 * included, is that of pa_slot_mapping + pa_quantize_and_cache + pa_decode.
 * Other quantised forms (per-block scales, head_dim 64, the vector-ALU
 * kernel) give PA_ERR_UNSUPPORTED: write them with pa_quantize_and_cache
 * first.
 *
 * Several query rows per sequence (chunked prefill, or checking several
 * drafted tokens in one pass: "Cache KV en production", section "Les
 * leviers"; forum thread, answer on chunked prefill): with query_start_loc
 * (device int32 [num_seqs + 1], 0 = query_start_loc[0] <= ... <=
 * query_start_loc[num_seqs] = num_queries), q and out are
 * [num_queries][num_q_heads][head_dim] and rows query_start_loc[s] ..
 * query_start_loc[s+1]-1 are the last L_s tokens of sequence s, already in
 * the cache and counted in context_lens[s] = n.  Row i of them sits at
 * position n - L_s + i and attends causally to positions 0 .. n - L_s + i
 * (a row that would see no token gets zeros).  max_query_len (host) bounds
 * L_s; rows whose index falls outside [0, num_queries) (offsets that do not
 * match num_queries, a caller error) are neither read nor written.
 * Matrix-core kernel only (bf16 queries with a bf16, int8 or E4M3 cache);
 * no fused cache write.
 *
 * Shared prefix (optional): when every sequence's first shared_prefix_len
 * tokens are the blocks shared_prefix_table[0 .. shared_prefix_len/BS - 1]
 * (a common prompt stored once: glossary, section 3, scenario 01; ia-vox,
 * prefix sharing), passing them lets the call read those blocks once for
 * the whole batch instead of once per sequence (with at most 16 query
 * heads per kv head; more are read through each table row).  The result
 * is the same
 * attention; a sequence shorter than the prefix sees only its own length
 * of it.  The caller guarantees that every table row starts with these
 * blocks.  With new_key/new_value, a sequence whose newest token lies
 * inside the prefix (context_lens[s] <= shared_prefix_len) has its row
 * neither stored nor attended (a shared block is never written; its
 * cached token is used), whichever kernel runs.  The matrix-core kernel
 * with one query row per sequence reads the prefix once for the batch; the
 * vector-ALU kernel and several query rows per sequence read it through
 * each table row as usual.  A given partition_tokens then sets the
 * partition length of both the prefix and the per-sequence part.
 * shared_prefix_table is a device int32 array (4-byte aligned).
 *
 * `kernel` selects the implementation: 0 = automatic, 1 = vector-ALU
 * kernel (any supported case), 2 = matrix-core kernel (bf16 queries with a
 * bf16, int8 or E4M3 cache, head_dim 64 or 128; else PA_ERR_UNSUPPORTED).
 * Both compute the definition above; they differ in rounding only.
 */
typedef struct {
  size_t struct_size;            /* = sizeof(pa_decode_args) */
  void* out;
  pa_dtype out_dtype;
  const void* q;
  pa_dtype q_dtype;
  void* k_cache;                 /* written only by the fused cache write */
  void* v_cache;
  pa_dtype kv_dtype;
  const float* k_scales;         /* non-NULL iff kv_dtype is PA_I8 or PA_FP8_E4M3 */
  const float* v_scales;
  const int32_t* block_tables;
  int32_t max_blocks_per_seq;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t max_context_len;       /* host-side bound on context_lens; sizes the grid */
  float scale;                   /* finite; usually 1/sqrt(head_dim) */
  int32_t partition_tokens;      /* 0 = automatic; else a multiple of 16, at most 128 * block_size */
  int32_t kernel;                /* 0 automatic, 1 vector ALU, 2 matrix cores */
  void* workspace;
  size_t workspace_bytes;
  void* stream;                  /* hipStream_t */
  const void* new_key;           /* optional fused cache write: both or neither */
  const void* new_value;
  int64_t total_context_len;     /* optional hint: sum of context_lens (0 = unknown), 0 <= it <= num_seqs * max_context_len */
  int32_t kv_scale_mode;         /* pa_scale_mode of k/v_scales (quantised caches; else ignored) */
  const int32_t* query_start_loc; /* NULL = one query row per sequence; else [num_seqs + 1] row offsets */
  int32_t num_queries;           /* with query_start_loc: total query rows (= query_start_loc[num_seqs]) */
  int32_t max_query_len;         /* with query_start_loc: host bound on the rows of one sequence, >= 1 */
  const int32_t* shared_prefix_table; /* optional: blocks of a prefix every sequence starts with */
  int32_t shared_prefix_len;     /* tokens of that prefix (multiple of block_size, <= max_context_len), 0 = none */
} pa_decode_args;

/* Host only: bytes of workspace pa_decode needs for these arguments
 * (device pointers are not read and may be NULL).  PA_ERR_INVALID /
 * PA_ERR_UNSUPPORTED as pa_decode would return. */
pa_status pa_decode_workspace_size(const pa_decode_args* a, size_t* bytes);

/* The same size as a plain return value: the bytes pa_decode_workspace_size
 * would store, or SIZE_MAX when it would return an error (pa_last_error()
 * then says which).  0 means no workspace is needed. */
size_t pa_decode_workspace_bytes(const pa_decode_args* a);

/* Launch decode attention as defined above. */
pa_status pa_decode(const pa_decode_args* a);

/* pa_decode for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the split-K workspace is a fixed array of
 * pa_decode_noalloc_scratch_bytes() bytes (64 MiB) that the library owns on
 * each GPU it runs on, held from the library's load until the process
 * ends.  a->workspace and a->workspace_bytes are ignored; everything else,
 * the result included, is as for pa_decode.  Arguments whose plan needs
 * more workspace than the array holds return PA_ERR_INVALID before any
 * launch.  The array's device address is looked up on the first call made
 * with each device current (the stream's device must be current, as for
 * any launch).  Every call on one GPU shares that GPU's array: calls that
 * may overlap on one GPU (two streams, two threads) race.  Calls no
 * hipMalloc or hipFree. */
pa_status pa_decode_noalloc(const pa_decode_args* a);
size_t pa_decode_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * Slot mapping: where each new token goes
 * ------------------------------------------------------------------------
 * slot_mapping[t] = block_tables[seq][pos / BS] * BS + pos % BS  (int64),
 * the flat slot of logical position pos of sequence seq (glossary figure,
 * section 2: token 40 of the table [7, 2, 11] lands in block 11, slot 8).
 *   seq = seq_idx[t], or t when seq_idx is NULL (then num_tokens must not
 *         exceed num_seqs);
 *   pos = positions[t], or context_lens[seq] - 1 (the newest token of a
 *         decode step) when positions is NULL.  Exactly one of positions
 *         and context_lens is non-NULL.
 * A negative position, a position past the table row, or a negative table
 * entry gives slot -1, which pa_reshape_and_cache skips.  Device arrays:
 * block_tables [num_seqs][max_blocks_per_seq], seq_idx / positions
 * [num_tokens] int32, context_lens [num_seqs] int32, slot_mapping
 * [num_tokens] int64 (written).
 */
pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t num_seqs, const int32_t* seq_idx, const int32_t* positions,
                          const int32_t* context_lens, int32_t num_tokens, int32_t block_size,
                          int64_t* slot_mapping, void* stream);

/* ------------------------------------------------------------------------
 * Cache write: scatter the new tokens' keys and values into their slots
 * ------------------------------------------------------------------------
 * For t < num_tokens with slot = slot_mapping[t] >= 0, for every kv head h:
 *   k_cache[slot / BS][h][slot % BS][:] = key[t][h][:]   (and value -> v_cache)
 * Bytes are copied unchanged; nothing else in the caches is written
 * ("Cache KV en production", section "Un cache par requête": the cache
 * grows by one token per decode step; K and V are never rewritten).
 * key, value [num_tokens][num_kv_heads][head_dim] of kv_dtype, caches as in
 * pa_decode, slot_mapping [num_tokens] int64.  Slots must be distinct and
 * below num_blocks * block_size (caller's responsibility).
 * Quantised caches are written with pa_quantize_and_cache; PA_I8 and
 * PA_FP8_E4M3 here are PA_ERR_UNSUPPORTED.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                               pa_dtype kv_dtype, const int64_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * Block copy for copy-on-write
 * ------------------------------------------------------------------------
 * For each pair p: (src, dst) = (block_pairs[2p], block_pairs[2p+1]), copy
 * the whole physical block -- all kv heads, all block_size slots -- of
 * k_cache and of v_cache from src to dst, and k_scales[src][:] /
 * v_scales[src][:] likewise when given (glossary, section 3, scenario 01:
 * shared pages are copied only when a sequence starts writing its own
 * tokens into them).  block_pairs is device int64 [num_pairs][2].  All ids
 * must lie in [0, num_blocks); destinations must be distinct and disjoint
 * from the sources (caller's responsibility), so the order of the pairs
 * does not matter.  Scales: non-NULL iff the cache is quantised, in the
 * layout scale_mode names (every scale of the block is copied).
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, pa_dtype kv_dtype, float* k_scales,
                         float* v_scales, int32_t scale_mode, const int64_t* block_pairs,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * Block swap between two pools (device <-> pinned host, or device <-> device)
 * ------------------------------------------------------------------------
 * For each pair p: (src, dst) = (block_pairs[2p], block_pairs[2p+1]), copy
 * the whole block src of the source pool (K, V, and the scales when given)
 * into block dst of the destination pool.  This moves a preempted or cold
 * request's blocks to CPU memory and back (ia-vox article, section
 * "Offloading et stratégies hybrides CPU/GPU"; "Cache KV en production":
 * a preempted request releases its pages and is restored later).  Both
 * pools have the shape [*][num_kv_heads][block_size][head_dim] of kv_dtype;
 * either may live in device memory or in pinned host memory allocated with
 * hipHostMalloc (the kernel reads and writes it over the host link).
 * block_pairs is device (or pinned host) int64 [num_pairs][2]; ids outside
 * [0, src_num_blocks) / [0, dst_num_blocks) skip the pair.  Destinations
 * must be distinct (caller's responsibility).  Scales: all four NULL, or
 * all four given for a quantised pool, in the layout scale_mode names.
 */
pa_status pa_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scales,
                         const float* src_v_scales, void* dst_k, void* dst_v, float* dst_k_scales,
                         float* dst_v_scales, pa_dtype kv_dtype, int32_t scale_mode,
                         const int64_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t src_num_blocks,
                         int32_t dst_num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * Quantising cache write (int8 or E4M3 caches)
 * ------------------------------------------------------------------------
 * The form of pa_reshape_and_cache for quantised caches (ia-vox article,
 * section "Quantization du KV cache": a fixed scale per layer, or one
 * recomputed for every token).  For t < num_tokens with slot =
 * slot_mapping[t] >= 0, for every kv head h, for K and V separately, in
 * fp32 with correctly rounded division:
 *   PA_SCALE_BLOCK (static): s = k_static_scale / v_static_scale (> 0,
 *     finite), stored as k_scales[b][h] / v_scales[b][h];
 *   PA_SCALE_TOKEN (dynamic): amax = max_d |x_d| of the row, s = amax / Q
 *     (Q = 127 for PA_I8, 448 for PA_FP8_E4M3; s = 1 when amax = 0),
 *     stored as k_scales[b][h][slot % BS];
 *   codes: PA_I8: clamp(rint(x_d / s), -127, 127), ties to even;
 *     PA_FP8_E4M3: the E4M3 code nearest to x_d / s, ties to the even
 *     mantissa, magnitudes above 448 saturating to 448, NaN to 0x7F.
 * key, value [num_tokens][num_kv_heads][head_dim] of src_dtype (PA_F32 or
 * PA_BF16); caches and scales as in pa_decode.  Slots must be distinct and
 * below num_blocks * block_size (caller's responsibility).
 */
pa_status pa_quantize_and_cache(const void* key, const void* value, pa_dtype src_dtype, void* k_cache,
                                void* v_cache, pa_dtype kv_dtype, float* k_scales, float* v_scales,
                                int32_t scale_mode, float k_static_scale, float v_static_scale,
                                const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostic: read-bandwidth probe (not part of attention)
 * ------------------------------------------------------------------------
 * Reads num_chunks chunks of chunk_bytes (1024, 2048 or 4096) bytes --
 * 4096 is one (block, kv head) of a bf16 cache with 16-token blocks and
 * head_dim 128, 2048 the same with 1-byte codes -- with the 16-byte
 * non-temporal loads the decode kernels use, and nothing else: chunk c is
 * base + chunk_bytes * c, or base + chunk_bytes * chunk_ids[c] when
 * chunk_ids (device int32 [num_chunks]) is given (for instance the chunks of a decode
 * batch in table order, which the block tables scatter over the pool).
 * num_waves waves of 64 lanes share the chunks; each stores one word per
 * lane into sink (device, num_waves * 64 uint32, written) so no load is
 * optimised away.  The caller guarantees every chunk lies inside one
 * allocation.  Used to measure the memory system's read ceiling for
 * decode's access pattern; the kernel's time over the bytes read is that
 * ceiling.
 */
pa_status pa_read_probe(const void* base, int64_t num_chunks, const int32_t* chunk_ids, int32_t chunk_bytes,
                        int32_t num_waves, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------
 * Block pool (host only)
 * ------------------------------------------------------------------------
 * A stack of free physical block ids with a reference count per block.
 * Blocks are taken page by page as sequences grow and go back to the
 * common pool as soon as no sequence holds them ("Cache KV en production",
 * section "PagedAttention : la pagination appliquée au cache KV"); a
 * cancelled request must return its blocks or they leak (glossary,
 * section 4); a shared prefix is held by several sequences at once
 * (glossary, section 3, scenario 01).
 *
 *  pa_pool_create: ids 0..num_blocks-1, all free; initial_order (host,
 *    NULL = 0, 1, 2, ...) is a permutation giving the order in which a
 *    fresh pool hands them out.  *out receives a pool the caller destroys.
 *  pa_block_alloc: all or nothing: PA_ERR_OOM (nothing changes) if fewer
 *    than n blocks are free; else pops n ids into out_ids (host, n
 *    entries), each with refcount 1.
 *  pa_block_share: refcount + 1 per entry of ids (host, n entries): one
 *    more sequence points at the block.
 *  pa_block_free: refcount - 1 per entry, in order; a block whose count
 *    reaches 0 is pushed back on the free stack at once (last freed is
 *    the next handed out).
 *  Share and free validate the whole call first: an id outside
 *  [0, num_blocks) is PA_ERR_INVALID (reported before any other error);
 *  sharing a free block, or freeing a block more times than it is held,
 *  is PA_ERR_STATE; nothing changes on error.  n = 0 is a no-op; n < 0 is
 *  PA_ERR_INVALID.
 */
typedef struct pa_pool pa_pool;

pa_status pa_pool_create(int32_t num_blocks, const int32_t* initial_order, pa_pool** out);
void pa_pool_destroy(pa_pool* p);
pa_status pa_block_alloc(pa_pool* p, int32_t n, int32_t* out_ids);
pa_status pa_block_share(pa_pool* p, int32_t n, const int32_t* ids);
pa_status pa_block_free(pa_pool* p, int32_t n, const int32_t* ids);
/* Reference count of block id, or -1 if id is out of range or p is NULL. */
int32_t pa_block_refcount(const pa_pool* p, int32_t id);
/* Number of free blocks, or -1 if p is NULL. */
int32_t pa_pool_num_free(const pa_pool* p);
int32_t pa_pool_num_blocks(const pa_pool* p);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
