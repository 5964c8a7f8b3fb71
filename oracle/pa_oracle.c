/*
 * pa_oracle.c -- CPU oracle for paged-KV-cache decode attention and its
 * companion cache operations.  TEST INFRASTRUCTURE ONLY: it is called from
 * tests, from the smoke check and from the CPU-baseline leg of the benchmark,
 * never from the product library, and it shares no code with it.
 *
 * Everything here is the plain definition, written for a reader to check by
 * eye: a naive gather of each logical token through the block table, then
 * attention in double precision.  No blocking, no fusion, no reordering.
 * OpenMP only distributes independent (sequence, query head) rows.
 *
 * Sources (the web pages this method is taken from):
 *  - "Cache KV en production" (blog), opening section: the current token's
 *    query is compared with the keys of every earlier token, and the result
 *    weights their values; K and V of a processed token never change.
 *  - deeplearn.tn KV-cache article, section "La taille réelle du cache KV":
 *    when predicting the next token only the last row of the attention is
 *    needed, so only the new token's query enters the computation.
 *  - "PagedAttention & Gestion du KV-Cache" glossary, section 2 (ASCII figure):
 *    logical blocks of 16 tokens map through a block table to physical blocks
 *    scattered in device memory (logical 0 -> 7, 1 -> 2, 2 -> 11).
 *  - "Cache KV en production", section "PagedAttention : la pagination
 *    appliquée au cache KV": fixed-size pages, one table per sequence from
 *    logical position to physical page, pages taken page by page.
 *
 * Element types (codes shared only by convention with the callers):
 *   0 = IEEE fp32, 1 = bfloat16 (upper 16 bits of an fp32), 2 = int8,
 *   3 = fp8 E4M3 in the OCP 8-bit floating-point format (1 sign bit, 4
 *       exponent bits with bias 7, 3 mantissa bits; no infinities, the
 *       all-ones exponent and mantissa encode NaN; largest finite 448).
 * Every stored element is converted to the double with the same value,
 * which is exact for all four types.
 *
 * Quantised caches (int8, fp8) carry fp32 scales in one of two layouts:
 *   scale mode 0: one scale per (block, KV head), [NB][Hkv];
 *   scale mode 1: one scale per (block, KV head, slot) = per token, [NB][Hkv][BS].
 * (ia-vox KV-cache article, section "Quantization du KV cache": a fixed
 * scale per layer is the static form, a scale recomputed for every token the
 * dynamic form.)
 *
 * Parity pins for every function live in tests/test_oracle_*.py; the
 * functions here have no "parity unpinned" part.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define OR_F32 0
#define OR_BF16 1
#define OR_I8 2
#define OR_FP8 3

#define OR_SCALE_BLOCK 0
#define OR_SCALE_TOKEN 1

/* ---- element decoding (input format, not the method) ------------------ */

/* Value of an OCP E4M3 code: sign, exponent field e, mantissa field m.
 * e == 0 is subnormal: m/8 * 2^(1-7); e in 1..15 is (1 + m/8) * 2^(e-7),
 * except e == 15 with m == 7, which is NaN. */
double oracle_fp8_e4m3_value(uint8_t code) {
  int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m / 8.0, 1 - 7);
  else v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

static double elem_as_double(const void* base, int64_t idx, int dtype) {
  if (dtype == OR_F32) {
    float f;
    memcpy(&f, (const char*)base + 4 * idx, 4);
    return (double)f;
  }
  if (dtype == OR_BF16) {
    uint16_t h;
    uint32_t bits;
    float f;
    memcpy(&h, (const char*)base + 2 * idx, 2);
    bits = ((uint32_t)h) << 16; /* bfloat16 is the top half of an fp32 */
    memcpy(&f, &bits, 4);
    return (double)f;
  }
  if (dtype == OR_FP8) return oracle_fp8_e4m3_value(((const uint8_t*)base)[idx]);
  /* int8 */
  return (double)((const int8_t*)base)[idx];
}

/* Threads the decode loop may use (OpenMP's current maximum). */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_elem_bytes(int dtype) {
  if (dtype == OR_F32) return 4;
  if (dtype == OR_BF16) return 2;
  if (dtype == OR_I8 || dtype == OR_FP8) return 1;
  return -1;
}

/* ---- gather through the block table ----------------------------------- */

/* Physical location of logical token t of sequence s: the table row of s,
 * entry t / BS, slot t % BS inside that block (glossary figure, section 2).
 * Returns the physical block id, or -1 when the table entry is unusable. */
static int64_t physical_block(const int32_t* block_tables, int max_blocks,
                              int s, int t, int BS, int NB) {
  int logical_block = t / BS;
  int32_t b;
  if (logical_block >= max_blocks) return -1;
  b = block_tables[(int64_t)s * max_blocks + logical_block];
  if (b < 0 || b >= NB) return -1;
  return b;
}

/* Flat element index of cache[b][g][slot][d] in the [NB][Hkv][BS][D] layout. */
static int64_t cache_index(int64_t b, int g, int slot, int d, int Hkv, int BS,
                           int D) {
  return (((b * Hkv + g) * BS) + slot) * (int64_t)D + d;
}

/* Index of the scale that applies to cache[b][g][slot][:]. */
static int64_t scale_index(int64_t b, int g, int slot, int Hkv, int BS, int scale_mode) {
  return scale_mode == OR_SCALE_TOKEN ? (b * Hkv + g) * BS + slot : b * Hkv + g;
}

/* One key or value component of token t, dequantised when the cache holds
 * int8 or fp8 codes: the stored code's value times its fp32 scale.  The
 * product of an fp32 and an int8 or E4M3 value is exact in double. */
static double kv_value(const void* cache, const float* scales, int dtype,
                       int scale_mode, int64_t b, int g, int slot, int d,
                       int Hkv, int BS, int D) {
  double x = elem_as_double(cache, cache_index(b, g, slot, d, Hkv, BS, D), dtype);
  if (dtype == OR_I8 || dtype == OR_FP8)
    x *= (double)scales[scale_index(b, g, slot, Hkv, BS, scale_mode)];
  return x;
}

/* ---- decode attention -------------------------------------------------- */

/*
 * out[r][h][:] = sum_t softmax_t(scale * <q[r][h], K_s[t]>) * V_s[t]
 * with query head h reading KV head h / (Hq / Hkv) (grouped-query heads in
 * contiguous groups).
 *
 * Decode (query_start_loc NULL): one query row per sequence, r = s, over
 * t = 0 .. context_lens[s]-1.
 * Several query rows per sequence (query_start_loc non-NULL, S + 1
 * offsets from 0): rows query_start_loc[s] .. query_start_loc[s+1]-1 are the last
 * L = query_start_loc[s+1] - query_start_loc[s] tokens of sequence s, whose
 * context length n counts them; row i of them sits at position n - L + i
 * and attends causally to t = 0 .. n - L + i (chunked prefill, and the
 * checking of several drafted tokens in one pass: "Cache KV en
 * production", section "Les leviers"; forum thread, answer on chunked
 * prefill).  A row with nothing to attend to gets zeros.
 *
 * All arithmetic in double; exp() from libm.  Returns 0, or -1 if some
 * table entry a sequence needs is outside [0, NB), a context length exceeds
 * max_blocks * BS, or the offsets do not start at 0 or decrease (nothing is read out of bounds
 * in that case; out is left partially written).
 */
int oracle_paged_attention(double* out, const void* q, int q_dtype,
                           const void* k_cache, const void* v_cache, int kv_dtype,
                           const float* k_scales, const float* v_scales,
                           int scale_mode, const int32_t* block_tables, int max_blocks,
                           const int32_t* context_lens, const int32_t* query_start_loc,
                           int S, int Hq, int Hkv, int D, int BS, int NB, double scale) {
  int G, bad = 0;
  int64_t row, R;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || BS <= 0 || Hq % Hkv) return -1;
  G = Hq / Hkv;
  if (query_start_loc && query_start_loc[0] != 0) return -1;
  for (int s = 0; s < S; ++s) {
    if (context_lens[s] < 0 || context_lens[s] > (int64_t)max_blocks * BS) return -1;
    if (query_start_loc && query_start_loc[s + 1] < query_start_loc[s]) return -1;
  }
  R = query_start_loc ? (int64_t)query_start_loc[S] : S;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (row = 0; row < R * Hq; ++row) {
    int r = (int)(row / Hq), h = (int)(row % Hq), g = h / G;
    int s = r, n, L = 1, i = 0;
    if (query_start_loc) { /* the sequence holding query row r */
      s = 0;
      while (query_start_loc[s + 1] <= r) ++s;
      L = query_start_loc[s + 1] - query_start_loc[s];
      i = r - query_start_loc[s];
    }
    /* tokens visible to this row: positions 0 .. n - L + i */
    n = context_lens[s] - L + i + 1;
    if (n > context_lens[s]) n = context_lens[s];
    if (n < 0) n = 0;
    const int64_t qoff = row * D;
    double* o = out + row * D;
    double* x;
    double m, z;
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (n == 0) continue;
    x = (double*)malloc(sizeof(double) * (size_t)n);
    /* scores x_t = scale * q . K_t */
    for (int t = 0; t < n; ++t) {
      int64_t b = physical_block(block_tables, max_blocks, s, t, BS, NB);
      double dot = 0.0;
      if (b < 0) { bad = 1; x[t] = 0.0; continue; }
      for (int d = 0; d < D; ++d)
        dot += elem_as_double(q, qoff + d, q_dtype) *
               kv_value(k_cache, k_scales, kv_dtype, scale_mode, b, g, t % BS, d, Hkv, BS, D);
      x[t] = scale * dot;
    }
    /* softmax weights exp(x_t - max x) / sum */
    m = x[0];
    for (int t = 1; t < n; ++t) if (x[t] > m) m = x[t];
    z = 0.0;
    for (int t = 0; t < n; ++t) { x[t] = exp(x[t] - m); z += x[t]; }
    /* weighted sum of the values */
    for (int t = 0; t < n; ++t) {
      int64_t b = physical_block(block_tables, max_blocks, s, t, BS, NB);
      double w = x[t] / z;
      if (b < 0) continue;
      for (int d = 0; d < D; ++d)
        o[d] += w * kv_value(v_cache, v_scales, kv_dtype, scale_mode, b, g, t % BS, d, Hkv, BS, D);
    }
    free(x);
  }
  return bad ? -1 : 0;
}

/* Decode: one query row per sequence. */
int oracle_paged_decode(double* out, const void* q, int q_dtype,
                        const void* k_cache, const void* v_cache, int kv_dtype,
                        const float* k_scales, const float* v_scales,
                        int scale_mode, const int32_t* block_tables, int max_blocks,
                        const int32_t* context_lens, int S, int Hq, int Hkv,
                        int D, int BS, int NB, double scale) {
  return oracle_paged_attention(out, q, q_dtype, k_cache, v_cache, kv_dtype, k_scales, v_scales, scale_mode,
                                block_tables, max_blocks, context_lens, NULL, S, Hq, Hkv, D, BS, NB, scale);
}

/* ---- slot mapping -------------------------------------------------------- */

/*
 * slot[t] = table[seq][pos / BS] * BS + pos % BS for the token at logical
 * position pos of sequence seq (glossary figure: logical block -> physical
 * block; "Cache KV en production": a table from each logical position to a
 * page).  seq is seq_idx[t], or t itself when seq_idx is NULL.  A negative
 * position, a position past the table row, or a negative table entry gives
 * slot -1 ("no write").
 */
void oracle_slot_mapping(int64_t* slots, const int32_t* block_tables,
                         int max_blocks, const int32_t* seq_idx,
                         const int32_t* positions, int T, int BS) {
  for (int t = 0; t < T; ++t) {
    int seq = seq_idx ? seq_idx[t] : t;
    int pos = positions[t];
    int32_t b;
    slots[t] = -1;
    if (pos < 0 || pos / BS >= max_blocks) continue;
    b = block_tables[(int64_t)seq * max_blocks + pos / BS];
    if (b < 0) continue;
    slots[t] = (int64_t)b * BS + pos % BS;
  }
}

/* ---- cache writes ---------------------------------------------------------- */

/*
 * Scatter of each new token's key and value into its slot
 * ("Cache KV en production", section "Un cache par requête": every decode
 * step grows the request's cache by one token).  key/value are [T][Hkv][D];
 * caches are [NB][Hkv][BS][D]; elements are copied as bytes.  Tokens are
 * applied in order; slot < 0 skips the token.  Returns -1 (after applying
 * the valid prefix) if a slot lies beyond the pool.
 */
int oracle_reshape_and_cache(const uint8_t* key, const uint8_t* value,
                             uint8_t* k_cache, uint8_t* v_cache, int elem_bytes,
                             const int64_t* slots, int T, int Hkv, int D,
                             int BS, int NB) {
  for (int t = 0; t < T; ++t) {
    int64_t slot = slots[t], b;
    int off;
    if (slot < 0) continue;
    b = slot / BS;
    off = (int)(slot % BS);
    if (b >= NB) return -1;
    for (int h = 0; h < Hkv; ++h)
      for (int d = 0; d < D; ++d) {
        int64_t src = ((int64_t)t * Hkv + h) * D + d;
        int64_t dst = cache_index(b, h, off, d, Hkv, BS, D);
        memcpy(k_cache + dst * elem_bytes, key + src * elem_bytes, (size_t)elem_bytes);
        memcpy(v_cache + dst * elem_bytes, value + src * elem_bytes, (size_t)elem_bytes);
      }
  }
  return 0;
}

/*
 * Copy-on-write block copy ("PagedAttention & Gestion du KV-Cache", section
 * 3, scenario 01: shared pages are duplicated only when a user starts to
 * produce its own continuation).  For each pair (src, dst), in order, the
 * whole physical block -- every KV head, every slot, used or not -- of the K
 * cache and of the V cache is copied, and so are the block's scales (all
 * of them in either scale layout) when the caller passes them.  Returns -1
 * (after applying the valid prefix) if an id lies outside [0, NB).
 */
int oracle_copy_blocks(uint8_t* k_cache, uint8_t* v_cache, int elem_bytes,
                       float* k_scales, float* v_scales, int scale_mode,
                       const int64_t* pairs, int P, int Hkv, int D, int BS, int NB) {
  const int64_t block_bytes = (int64_t)Hkv * BS * D * elem_bytes;
  const int64_t nsc = scale_mode == OR_SCALE_TOKEN ? (int64_t)Hkv * BS : Hkv;
  for (int p = 0; p < P; ++p) {
    int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= NB || dst < 0 || dst >= NB) return -1;
    memmove(k_cache + dst * block_bytes, k_cache + src * block_bytes, (size_t)block_bytes);
    memmove(v_cache + dst * block_bytes, v_cache + src * block_bytes, (size_t)block_bytes);
    if (k_scales)
      for (int64_t i = 0; i < nsc; ++i) k_scales[dst * nsc + i] = k_scales[src * nsc + i];
    if (v_scales)
      for (int64_t i = 0; i < nsc; ++i) v_scales[dst * nsc + i] = v_scales[src * nsc + i];
  }
  return 0;
}

/*
 * Block swap between two pools of the same shape (ia-vox article, section
 * "Offloading et stratégies hybrides CPU/GPU": cold parts of the cache move
 * to CPU memory and back; "Cache KV en production": a preempted request's
 * pages are released and its state restored later).  For each pair
 * (src, dst), the whole block src of the source pool (K, V and, when given,
 * its scales) is copied to block dst of the destination pool.  Returns -1
 * (after applying the valid prefix) if an id lies outside its pool.
 */
int oracle_swap_blocks(const uint8_t* src_k, const uint8_t* src_v,
                       const float* src_ks, const float* src_vs,
                       uint8_t* dst_k, uint8_t* dst_v, float* dst_ks,
                       float* dst_vs, int elem_bytes, int scale_mode,
                       const int64_t* pairs, int P, int Hkv, int D, int BS,
                       int src_NB, int dst_NB) {
  const int64_t block_bytes = (int64_t)Hkv * BS * D * elem_bytes;
  const int64_t nsc = scale_mode == OR_SCALE_TOKEN ? (int64_t)Hkv * BS : Hkv;
  for (int p = 0; p < P; ++p) {
    int64_t src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= src_NB || dst < 0 || dst >= dst_NB) return -1;
    memcpy(dst_k + dst * block_bytes, src_k + src * block_bytes, (size_t)block_bytes);
    memcpy(dst_v + dst * block_bytes, src_v + src * block_bytes, (size_t)block_bytes);
    if (src_ks && dst_ks)
      for (int64_t i = 0; i < nsc; ++i) dst_ks[dst * nsc + i] = src_ks[src * nsc + i];
    if (src_vs && dst_vs)
      for (int64_t i = 0; i < nsc; ++i) dst_vs[dst * nsc + i] = src_vs[src * nsc + i];
  }
  return 0;
}

/* ---- int8 quantiser -------------------------------------------------------- */

/*
 * Symmetric int8 quantisation with one fp32 scale per (block, KV head)
 * (ia-vox KV-cache article, section "Quantization du KV cache": a scale per
 * layer is the static form and a scale per token the dynamic form; this is
 * the per-block form in between).  Over the valid slots of a (block, head):
 *   amax = max |x|;  s = amax / 127 (fp32, round to nearest);
 *   code = clamp(rint(x / s), -127, 127) with x / s in fp32 and rint
 *   rounding half to even;  amax == 0 gives s = 1 and codes 0.
 * Slots at or past valid[b] get code 0.  x and codes are [NB][Hkv][BS][D],
 * scales [NB][Hkv].
 */
void oracle_quantize_int8(int8_t* codes, float* scales, const float* x,
                          const int32_t* valid, int NB, int Hkv, int BS, int D) {
  for (int64_t b = 0; b < NB; ++b)
    for (int g = 0; g < Hkv; ++g) {
      float amax = 0.0f, s;
      int n = valid[b] < BS ? valid[b] : BS;
      for (int t = 0; t < n; ++t)
        for (int d = 0; d < D; ++d) {
          float a = fabsf(x[cache_index(b, g, t, d, Hkv, BS, D)]);
          if (a > amax) amax = a;
        }
      s = amax > 0.0f ? amax / 127.0f : 1.0f;
      scales[b * Hkv + g] = s;
      for (int t = 0; t < BS; ++t)
        for (int d = 0; d < D; ++d) {
          int64_t i = cache_index(b, g, t, d, Hkv, BS, D);
          float r;
          if (t >= n || amax == 0.0f) { codes[i] = 0; continue; }
          r = rintf(x[i] / s);
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          codes[i] = (int8_t)r;
        }
    }
}

/* ---- quantising cache write -------------------------------------------- */

/*
 * Nearest E4M3 code to the fp32 value v: the finite code whose value is
 * closest to v; between two equally close codes the one with an even
 * mantissa field; |v| beyond the largest finite value (448) gives +-448
 * (saturation); NaN gives the NaN code 0x7F.  The non-negative finite
 * codes 0..0x7E have strictly increasing values, so the search bisects for
 * the last code whose value does not exceed |v| and compares it with the
 * next code up.
 */
uint8_t oracle_fp8_e4m3_encode(float v) {
  const int sign = signbit(v) ? 1 : 0;
  const double a = fabs((double)v);
  int best;
  if (isnan(v)) return 0x7F;
  if (a >= 448.0) {
    best = 0x7E;
  } else {
    /* value(lo) <= a < value(hi) throughout */
    int lo = 0, hi = 0x7E;
    double below, above;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (oracle_fp8_e4m3_value((uint8_t)mid) <= a)
        lo = mid;
      else
        hi = mid;
    }
    below = a - oracle_fp8_e4m3_value((uint8_t)lo);
    above = oracle_fp8_e4m3_value((uint8_t)hi) - a;
    best = (above < below || (above == below && (hi & 1) == 0)) ? hi : lo;
  }
  return (uint8_t)(best | (sign << 7));
}

/* One element in the source format as an fp32 value (exact). */
static float src_as_float(const void* base, int64_t idx, int dtype) {
  return (float)elem_as_double(base, idx, dtype);
}

/*
 * Quantising form of the cache write: each new token's key and value rows
 * ([T][Hkv][D], fp32 or bf16) are stored as int8 or E4M3 codes with fp32
 * scales, tokens in order, slot < 0 skipped.  Per (token, KV head), for K
 * and V separately, in fp32:
 *   scale mode 0 (static, one scale for the layer): s = the caller's static
 *     scale, and scales[b][h] = s;
 *   scale mode 1 (dynamic, per token): amax = max_d |x_d|, s = amax / qmax
 *     (qmax = 127 for int8, 448 for E4M3), s = 1 when amax == 0, and
 *     scales[b][h][slot % BS] = s;
 *   code_d = int8: clamp(rint(x_d / s), -127, 127), rint rounding half to
 *     even; E4M3: the nearest code to x_d / s (oracle_fp8_e4m3_encode).
 * Returns -1 (after applying the valid prefix) if a slot lies beyond the
 * pool or the static scale is not positive and finite.
 */
int oracle_quantize_and_cache(const void* key, const void* value, int src_dtype,
                              void* k_cache, void* v_cache, int kv_dtype,
                              float* k_scales, float* v_scales, int scale_mode,
                              float k_static, float v_static,
                              const int64_t* slots, int T, int Hkv, int D,
                              int BS, int NB) {
  const float qmax = kv_dtype == OR_FP8 ? 448.0f : 127.0f;
  if (scale_mode == OR_SCALE_BLOCK &&
      !(k_static > 0.0f && v_static > 0.0f && isfinite(k_static) && isfinite(v_static)))
    return -1;
  for (int t = 0; t < T; ++t) {
    int64_t slot = slots[t], b;
    int off;
    if (slot < 0) continue;
    b = slot / BS;
    off = (int)(slot % BS);
    if (b >= NB) return -1;
    for (int h = 0; h < Hkv; ++h)
      for (int kv = 0; kv < 2; ++kv) {
        const void* src = kv ? value : key;
        void* cache = kv ? v_cache : k_cache;
        float* scales = kv ? v_scales : k_scales;
        const int64_t row = ((int64_t)t * Hkv + h) * D;
        float s;
        if (scale_mode == OR_SCALE_BLOCK) {
          s = kv ? v_static : k_static;
        } else {
          float amax = 0.0f;
          for (int d = 0; d < D; ++d) {
            float a = fabsf(src_as_float(src, row + d, src_dtype));
            if (a > amax) amax = a;
          }
          s = amax > 0.0f ? amax / qmax : 1.0f;
        }
        scales[scale_index(b, h, off, Hkv, BS, scale_mode)] = s;
        for (int d = 0; d < D; ++d) {
          const float r = src_as_float(src, row + d, src_dtype) / s;
          const int64_t i = cache_index(b, h, off, d, Hkv, BS, D);
          if (kv_dtype == OR_FP8) {
            ((uint8_t*)cache)[i] = oracle_fp8_e4m3_encode(r);
          } else {
            float c = rintf(r);
            if (c > 127.0f) c = 127.0f;
            if (c < -127.0f) c = -127.0f;
            ((int8_t*)cache)[i] = (int8_t)c;
          }
        }
      }
  }
  return 0;
}
