// Paged decode attention for gfx950.
//
// What is computed (the definition restated in pa.h): for each sequence s
// and query head h, the newest token's query attends over the n tokens of
// its sequence, which a block table scatters over fixed-size physical
// blocks ("Cache KV en production", opening section and section on paging;
// glossary "PagedAttention & Gestion du KV-Cache", section 2 figure).
// Decode reads every cached key and value once per step and does little
// arithmetic per byte, so it is bound by HBM bandwidth (forum thread, post
// of 17:05; deeplearn.tn article, section "Le compromis fondamental").
//
// Work decomposition: one wave per (sequence, kv head, partition of the
// context); the partition's tokens are processed in tiles of 16.  With
// more than one partition each wave leaves (m, l, acc) in the workspace and
// decode_merge_kernel combines them; with one partition the wave writes the
// output row directly.
//
// Softmax bookkeeping is in log2 units: x = log2(e) * scale * <q, k>, weights
// exp2(x - m).  m is a per-head reference value, moved only when a score
// exceeds it by more than kRescaleThreshold (results are exact for any
// reference; the threshold bounds weights by 2^8 and makes rescaling of
// the accumulators rare).
#include <type_traits>

#include "pa_internal.h"
#include "pa_quant.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleThreshold = 8.0f;
constexpr float kNegInf = -__builtin_huge_valf();
// A finite starting reference (log2 units), the lowest finite float: any
// larger finite score exceeds it by more than kRescaleThreshold (8 is below
// its spacing), so the first one moves the reference, and
// 2^(-inf - kFloorRef) = 0.
constexpr float kFloorRef = -3.40282347e38f;

// Streaming loads: every cached byte is read once per step, so they bypass
// reuse in the caches (non-temporal hint).
__device__ __forceinline__ u32x4_t ld16(const void* p) { return __builtin_nontemporal_load((const u32x4_t*)p); }
__device__ __forceinline__ u32x2_t ld8(const void* p) { return __builtin_nontemporal_load((const u32x2_t*)p); }
__device__ __forceinline__ unsigned ld4(const void* p) { return __builtin_nontemporal_load((const unsigned*)p); }

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
// signed byte k of w as float
__device__ __forceinline__ float i8_at(unsigned w, int k) { return (float)(int)(signed char)(w >> (8 * k)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Settle a loaded value before a loop: an empty asm statement that takes the
// register as input and output emits nothing, but the compiler waits for
// the load once, here, and inside the loop the value is no longer a load in
// flight.  (Otherwise its wait analysis, merging the states around the loop,
// keeps re-waiting with vmcnt(0) -- for every load, the next tiles'
// prefetches included -- before each use in every iteration.)
template <typename T>
__device__ __forceinline__ void settle(T& x) {
  asm volatile("" : "+v"(x));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}

// Reductions across the four 16-lane rows (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap instructions: permlane16_swap exchanges odd and even
// rows, permlane32_swap the two wave halves; combining both returned copies
// gives every lane the result for its column.
__device__ __forceinline__ float swap16_max(float x) {
  const u32x2_t r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                                                                  __float_as_uint(x), false, false));
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
  const u32x2_t r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                                                  __float_as_uint(x), false, false));
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
  const u32x2_t r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                                                                  __float_as_uint(x), false, false));
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const u32x2_t r = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                                                  __float_as_uint(x), false, false));
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor_max_rows(float x) { return swap32_max(swap16_max(x)); }
__device__ __forceinline__ float xor_sum_rows(float x) { return swap32_sum(swap16_sum(x)); }

__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false)));
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false)));
}
__device__ __forceinline__ float wave_max(float x) { return xor_max_rows(row_max16(x)); }

template <bool FP8>
__device__ __forceinline__ u32x2_t quant_row8(u32x4_t w, float& scale) {
  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = row_max16(amax);
  const float s = amax > 0.f ? amax / quant_max<FP8>() : 1.f;
  unsigned lo = 0u, hi = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo |= quant_code<FP8>(x[e] / s) << (8 * e);
    hi |= quant_code<FP8>(x[4 + e] / s) << (8 * e);
  }
  scale = s;
  return u32x2_t{lo, hi};
}
__device__ __forceinline__ float wave_sum(float x) { return xor_sum_rows(row_sum16(x)); }

// ---------------------------------------------------------------------------
// Split-K partials.  With more than one partition every wave that attended
// to some tokens stores (m, l, acc) in the workspace; decode_merge_kernel
// then combines each row's partials in partition order:
//   out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p,  M = max_p m_p.
// (A merge fused into the last-arriving wave needs an agent-scope release
// per wave, which on gfx950 writes back the XCD's L2; measured 70 us slower
// per 70B-shaped layer than this separate launch.)
// ---------------------------------------------------------------------------

struct SplitK {
  float2* ml;     // [S][Hq][nP]: reference max (log2 units), sum of weights
  float* acc;     // [S][Hq][nP][D]: unnormalised weighted sum of values
  int32_t* counts;  // balanced split: partials of each sequence [S], else NULL
};

// One workgroup of W waves per output row (query row, head): out = sum_p
// 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p over the partitions that hold
// tokens, in partition order.  Every partition of the grid leaves its
// (m, l), empty ones (-inf, 0), so a row's nP partials can be read without
// first reading its length (a balanced split instead records how many
// partials each sequence has, and only those are read).  With lengths given (decode rows) and W > 1
// (long ragged rows, most partitions empty) only the ceil(n / P) that hold
// tokens are read.  Partitions are read sixteen at a time, all loads of a
// group issued together (one memory round trip per group); wave w takes
// groups w, w + W, ...; groups after a wave's first rescale its running
// sums to the new maximum.  With W > 1 the waves' (m, L, acc) are combined
// through LDS the same way, in wave order.  W = 1 when every row has at
// most 16 partitions; plans with up to 32, 64 or more partitions get W = 2,
// 4 or 8, so a long ragged row needs about one round trip per wave.
template <int D, int W>
__global__ __launch_bounds__(64 * W) void decode_merge_kernel(float* __restrict__ out, SplitK ws,
                                                              const int32_t* __restrict__ context_lens, int Hq,
                                                              int P, int nP, int max_tokens) {
  constexpr int PER = D / 64;
  constexpr int GRP = 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const size_t row = blockIdx.x;
  int np = nP;
  if (ws.counts) {
    np = min(nP, max(0, ws.counts[row / Hq]));
  } else if (W > 1 && context_lens) {
    const int n = min(context_lens[row / Hq], max_tokens);
    np = n > 0 ? min(nP, (n + P - 1) / P) : 0;
  }
  // A row with at most GRP partials needs one wave: the others leave before
  // any barrier (the condition is the same for the whole workgroup).
  const bool solo = W > 1 && np <= GRP;
  if (solo && wave > 0) return;
  const size_t r = row * (size_t)nP;
  float m_run = kNegInf, L = 0.f, a[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) a[q] = 0.f;
  for (int p0 = GRP * wave; p0 < np; p0 += GRP * W) {
    const int cnt = min(GRP, np - p0);
    float part[GRP][PER];
    const float* src = ws.acc + (r + p0) * D + lane;
#pragma unroll
    for (int k = 0; k < GRP; ++k)
#pragma unroll
      for (int q = 0; q < PER; ++q) part[k][q] = k < cnt ? src[(size_t)k * D + 64 * q] : 0.f;
    const float2 v = lane < cnt ? ws.ml[r + p0 + lane] : float2{kNegInf, 0.f};
    const float mc = wave_max(v.y > 0.f ? v.x : kNegInf);
    const float m_new = fmaxf(m_run, mc);
    if (m_new == kNegInf) continue;  // no weight anywhere yet
    if (m_run != kNegInf && m_run != m_new) {
      const float alpha = fast_exp2(m_run - m_new);
      L *= alpha;
#pragma unroll
      for (int q = 0; q < PER; ++q) a[q] *= alpha;
    }
    m_run = m_new;
    const float w = (lane < cnt && v.y > 0.f) ? fast_exp2(v.x - m_new) : 0.f;
    L += wave_sum(w * v.y);
#pragma unroll
    for (int k = 0; k < GRP; ++k) {
      // an empty partition's acc row was never written: select, not multiply
      const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k));
#pragma unroll
      for (int q = 0; q < PER; ++q) a[q] = wk > 0.f ? fmaf(wk, part[k][q], a[q]) : a[q];
    }
  }
  if (W > 1 && !solo) {
    __shared__ float s_ml[W][2];
    __shared__ float s_a[W][D];
    if (lane == 0) {
      s_ml[wave][0] = m_run;
      s_ml[wave][1] = L;
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) s_a[wave][lane + 64 * q] = a[q];
    __syncthreads();
    if (wave != 0) return;
    float M = kNegInf;
#pragma unroll
    for (int u = 0; u < W; ++u) M = fmaxf(M, s_ml[u][0]);
    L = 0.f;
#pragma unroll
    for (int q = 0; q < PER; ++q) a[q] = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int u = 0; u < W; ++u) {
        const float mu = s_ml[u][0];
        const float f = mu == kNegInf ? 0.f : fast_exp2(mu - M);
        L += f * s_ml[u][1];
#pragma unroll
        for (int q = 0; q < PER; ++q) a[q] = fmaf(f, s_a[u][lane + 64 * q], a[q]);
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* o = out + row * D + lane;
#pragma unroll
  for (int q = 0; q < PER; ++q) o[64 * q] = a[q] * inv;
}

// ===========================================================================
// Matrix-core kernel: bf16 or int8 cache, bf16 queries, head_dim 128,
// up to 16 query heads per kv head.
//
// Per 16-token tile:
//  * scores S[t][h] = K[t][:] . q[h][:] with four v_mfma_f32_16x16x32_bf16:
//    A = K tile (row = token, read straight from HBM), B = the group's
//    queries (column = head; columns >= G hold zeros).  Lane l receives the
//    scores of head l%16 for tokens 4*(l/16) + r, r = 0..3.
//  * weights P = exp2(x - m) stay in fp32 and are split into bf16 hi + lo
//    parts so the P.V product keeps ~16 significant bits of P.
//  * O^T[d][h] += V^T[d][t] P^T[t][h] with v_mfma_f32_16x16x16bf16_1k: the
//    B operand is P in exactly the layout the score MFMA produced; the A
//    operand wants four tokens of one d per lane, which each lane builds
//    from its four 16-byte V rows with v_perm_b32 (no LDS round trip).
//    MFMA e (0..7) covers d = 8*c + e for c = 0..15, so lane l ends with
//    head l%16 and the 32 contiguous d = 32*(l/16) .. +31.
// ===========================================================================

template <int RB>
struct MfmaTile {
  // K, coalesced and staged through LDS into the MFMA layout, RB / 64
  // loads of 16 B per lane:
  //    256-byte rows (bf16, head_dim 128): instruction i reads rows
  //    4i .. 4i+3, lane l the 16 B chunk l%16 of row 4i + l/16;
  //    128-byte rows (1-byte codes at head_dim 128, bf16 at 64): rows
  //    8i .. 8i+7, lane l chunk l%8 of row 8i + l/8;
  //    64-byte rows (1-byte codes at head_dim 64): all 16 rows, lane l
  //    chunk l%4 of row l/4.
  u32x4_t k[RB / 64];
  // V: rows 4*(l/16) + i, the lane's sixteenth of the row (element run
  // l%16): 16, 8 or 4 B (the rest zero).
  u32x4_t v[4];
};

// A tile's loads are buffer loads: the tile's first row is the base of a
// scalar resource descriptor covering exactly the 16 rows, and each lane
// adds a constant byte offset (koff[i] / voff[i]) held in a register that is
// never rewritten, so no load ever has to wait for an earlier one to finish
// before its address can be formed.  An access past the 16 rows would read
// zeros instead of touching other memory.
constexpr int kBufferFormat = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, kBufferFormat);
}
// AUX: the loads' cache policy bits, 2 = non-temporal (streamed K/V, read
// once), 0 = normal (tiles that other waves read again soon)
template <int AUX = 2>
__device__ __forceinline__ u32x4_t bld16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX = 2>
__device__ __forceinline__ u32x2_t bld8(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
}
template <int AUX = 2>
__device__ __forceinline__ unsigned bld4(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX);
}

template <int RB, int AUX = 2>
__device__ __forceinline__ void mfma_load_tile(MfmaTile<RB>& T, const char* kbase, const char* vbase,
                                               const unsigned (&koff)[4], const unsigned (&voff)[4]) {
  constexpr int TILE = 16 * RB;  // bytes of 16 token rows
  const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kbase, TILE), rv = tile_rsrc(vbase, TILE);
#pragma unroll
  for (int i = 0; i < RB / 64; ++i) T.k[i] = bld16<AUX>(rk, koff[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (RB == 64) {
      T.v[i] = u32x4_t{bld4<AUX>(rv, voff[i]), 0u, 0u, 0u};
    } else if constexpr (RB == 128) {
      const u32x2_t w = bld8<AUX>(rv, voff[i]);
      T.v[i] = u32x4_t{w[0], w[1], 0u, 0u};
    } else {
      T.v[i] = bld16<AUX>(rv, voff[i]);
    }
  }
}

// int8 -> bf16 for 4 consecutive codes packed in w: exact (|code| <= 127 fits
// bf16's 8-bit significand), so the float's upper half is the bf16.
__device__ __forceinline__ u32x2_t i8x4_to_bf16x4(unsigned w) {
  const unsigned f0 = __float_as_uint(i8_at(w, 0)), f1 = __float_as_uint(i8_at(w, 1));
  const unsigned f2 = __float_as_uint(i8_at(w, 2)), f3 = __float_as_uint(i8_at(w, 3));
  return u32x2_t{__builtin_amdgcn_perm(f1, f0, 0x07060302u), __builtin_amdgcn_perm(f3, f2, 0x07060302u)};
}

// E4M3 -> bf16 for 4 consecutive codes packed in w: the hardware converts
// two codes at a time to fp32 (OCP E4M3, exact), and every E4M3 value fits
// bf16 exactly (3 mantissa bits, exponents 2^-9 .. 2^8), so the fp32's upper
// half is the bf16.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2_t e4m3x4_to_bf16x4(unsigned w) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  return u32x2_t{__builtin_amdgcn_perm(__float_as_uint(lo[1]), __float_as_uint(lo[0]), 0x07060302u),
                 __builtin_amdgcn_perm(__float_as_uint(hi[1]), __float_as_uint(hi[0]), 0x07060302u)};
}

// Cache element kinds of the matrix-core kernel.
constexpr int kKvBf16 = 0, kKvI8 = 1, kKvFp8 = 2;
template <int KV>
__device__ __forceinline__ u32x2_t codes_to_bf16x4(unsigned w) {
  if constexpr (KV == kKvFp8) return e4m3x4_to_bf16x4(w);
  else return i8x4_to_bf16x4(w);
}

// The fused quantising write: 8 bf16 values of a row (d = 8c .. 8c+7 in
// lane c of a 16-lane row; the 16 lanes hold the row of 128) -> their 8
// code bytes, and the row's per-token scale amax / quant_max, exactly as
// pa_quantize_and_cache computes them (the same row maximum, division and
// code function).
template <bool FP8>
__device__ __forceinline__ u32x2_t quant_row8(u32x4_t w, float& scale);

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }
__device__ __forceinline__ i16x4_t as_i16x4(unsigned a, unsigned b) {
  return __builtin_bit_cast(i16x4_t, u32x2_t{a, b});
}
// two floats to bf16 (round to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32 (two scalar conversions would take four instructions)
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Work item of a wave: (sequence s, kv head g, partition p[, column group
// cg]), kv head fastest: the waves that start together read neighbouring
// 4 KB chunks of the same physical blocks (measured ~1 % faster than
// partition fastest on the 70B-shaped layer; giving each XCD a contiguous
// range of items instead of the round-robin dispatch order measured no
// better).
__device__ __forceinline__ void mfma_item(int item, int Hkv, int nP, int CG, int& s, int& g, int& p, int& cg) {
  g = item % Hkv;
  const int rest = item / Hkv;
  cg = rest % CG;
  const int sp = rest / CG;
  p = sp % nP;
  s = sp / nP;
}

// A shared prefix (cascade): the first items of the grid attend every
// sequence's query row to the blocks of one shared table -- a "virtual
// sequence" whose columns are (sequence, head) pairs, 16 per column group,
// each lane masking to its own sequence's length -- so each prefix K/V tile
// is read once per column group instead of once per sequence; the other
// items attend each sequence to its tokens from t0 = prefix length on.
// Both write partials: prefix partition p at slot p, the sequence's
// partition p at slot nPp + p, of nPw slots per row.  An item of a cascade
// launch is a workgroup of kCascadeWaves waves: wave w takes tiles
// tile_begin + w, tile_begin + w + kCascadeWaves, ... of the partition
// (chains a quarter as long, the neighbouring tiles in flight together)
// and the waves' (m, l, acc)
// are combined through LDS before the one partial is written.
struct Cascade {
  const int32_t* table;  // shared prefix blocks (NULL: no prefix items)
  int blocks;            // prefix length / BS
  int items;             // prefix items = Hkv * nP * CG, first in the grid
  int nP, P, CG;         // prefix partitions, their length, column groups
  int t0;                // first token of the per-sequence items
  int nPw;               // partial slots per output row (1: write out directly)
  int write_from;        // fused write: positions below (a shared prefix) are neither stored nor taken from new_k
};

constexpr int kModeDecode = 0, kModeMultiQuery = 1, kModeCascade = 2, kModeBalanced = 3, kModeBalancedWide = 4;

// Balanced split of a ragged decode batch.  A kv head's work is the
// sequence of 16-token tiles of all sequences in order; it is cut into V
// ranges of pw tiles, range v handled by wave v mod Wh of the head (waves
// loop over their ranges).  A range that crosses sequence boundaries is
// processed as pieces, one per sequence, each leaving a partial in slot
// v - (first range of that sequence).  Every wave reads all lengths once
// (sequence 64*ch + lane in chunk ch of CH) and scans the tile counts; tile
// index a -> its sequence by a ballot over the inclusive sums.  CH = 4
// chunks (256 sequences) in the balanced mode, 16 (1,024) in the wide one.
constexpr int kBalancedChunks = kBalancedMaxSeqs / 64;
constexpr int kBalancedWideChunks = kBalancedWideMaxSeqs / 64;
template <int CH>
struct TileMap {
  int incl[CH];  // inclusive prefix sums of the tile counts
  int len[CH];   // the sequences' lengths (capped at the table row)
  int last[CH];  // incl of each chunk's last lane (wave-uniform)
  int total;     // tiles of all sequences
};

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// tiles attended of a sequence of n tokens: those of its first min(n, cap)
__device__ __forceinline__ int tile_count(int n, int cap) { return n > 0 ? (min(n, cap) + 15) >> 4 : 0; }

template <int CH>
__device__ __forceinline__ void tile_map_init(TileMap<CH>& m, const int32_t* __restrict__ context_lens, int S,
                                              int row_cap, int cap, int lane) {
  int n[CH];
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int si = 64 * ch + lane;
    n[ch] = si < S ? max(0, min(context_lens[si], row_cap)) : 0;
  }
  int run = 0;
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const int x = wave_incl_scan(tile_count(n[ch], cap), lane) + run;
    m.incl[ch] = x;
    m.len[ch] = n[ch];
    run = __builtin_amdgcn_readlane(x, 63);
    m.last[ch] = run;
  }
  m.total = run;
}

// tile index a < m.total -> sequence s, its length n, tile count c and the
// tiles before it (the chunk found by counting, its values by selects: no
// indexing of the register arrays)
template <int CH>
__device__ __forceinline__ void tile_find(const TileMap<CH>& m, int a, int cap, int& s, int& n, int& c, int& excl) {
  int ch = 0;
#pragma unroll
  for (int k = 0; k + 1 < CH; ++k) ch += m.last[k] <= a ? 1 : 0;
  int incl = m.incl[0], len = m.len[0];
#pragma unroll
  for (int k = 1; k < CH; ++k) {
    incl = ch == k ? m.incl[k] : incl;
    len = ch == k ? m.len[k] : len;
  }
  const unsigned long long b = __ballot(incl > a);
  const int l = b ? __builtin_ctzll(b) : 0;
  n = __builtin_amdgcn_readlane(len, l);
  c = tile_count(n, cap);
  excl = __builtin_amdgcn_readlane(incl, l) - c;
  s = 64 * ch + l;
}

struct Balanced {
  int min_tiles;  // least tiles per range (keeps every sequence's pieces within nP slots)
  int cap;        // tokens attended per sequence at most (max_context_len)
};
static_assert(kCascadeWaves == 1 || kCascadeWaves == 2 || kCascadeWaves == 4, "1, 2 or 4 waves per item");

// KV: kKvBf16, kKvI8 or kKvFp8 cache; TOKSC: quantised cache with one scale
// per token ([NB][Hkv][BS]) instead of one per (block, kv head).
//
// Columns of the MFMA B operand.  Decode (qsl == NULL): column c is query
// head g*G + c of the sequence's one query row.  Several causal query rows
// per sequence (qsl = row offsets): the sequence's L rows times G heads are
// numbered row-major, col = 16*cg + c -> (row i = col / G, head col % G),
// and column group cg takes 16 of them; row i sits at position n - L + i
// and sees tokens up to it, so each lane column masks its own limit.  A
// wave carries NCG consecutive column groups over the same K/V tiles (one
// score MFMA chain, softmax state and accumulator set per group, V^T
// operands built once), so K/V are read once per NCG groups.
//
// Waves per workgroup WG: one, except in the cascade mode (kCascadeWaves
// waves share each item, taking its tiles in turn) and in groups (decode or
// several query rows with one column group per item: one workgroup per
// (sequence, kv head), wave w taking partition w of at most WG; a wave
// whose partition is empty still joins the combination, with no weight).
// Either way the workgroup's waves combine (m, l, acc) through LDS and
// wave 0 goes on with the result, so a grouped launch writes the output
// rows itself: no partials, no merge.
template <int KV, int BS, bool TOKSC, int NCG, int MODE, int WG, int D>
__global__ __launch_bounds__(64 * WG) void decode_mfma_kernel(
    float* __restrict__ out, SplitK ws,
    const unsigned short* __restrict__ q, char* __restrict__ k_cache, char* __restrict__ v_cache,
    float* __restrict__ k_scales, float* __restrict__ v_scales, const int32_t* __restrict__ tables,
    int max_blocks, const int32_t* __restrict__ context_lens, int Hq, int Hkv, int G, int NB, float qk_log2,
    int P, int nP, const char* __restrict__ new_k, const char* __restrict__ new_v,
    const int32_t* __restrict__ qsl, int CG, int num_rows, Cascade cz, Balanced bz) {
  constexpr bool MQ = MODE == kModeMultiQuery;
  constexpr bool GROUP = WG > 1 && MODE != kModeCascade;
  constexpr bool BAL = MODE == kModeBalanced || MODE == kModeBalancedWide;
  constexpr int CH = MODE == kModeBalancedWide ? kBalancedWideChunks : kBalancedChunks;
  static_assert(MODE == kModeCascade ? WG == kCascadeWaves
                : BAL ? WG == 1
                                        : (WG == 1 || WG == 2 || WG == 4 || WG == 8) && (WG == 1 || NCG == 1),
                "waves per workgroup");
  constexpr int WPI = WG;                                // waves combined per workgroup
  constexpr int TS = MODE == kModeCascade ? WG : 1;      // tile stride of one wave
  constexpr bool I8 = KV != kKvBf16;  // 1-byte codes with fp32 scales
  constexpr int E = I8 ? 1 : 2;
  static_assert(D == 128 || D == 64, "head_dim 64 or 128");
  constexpr int KK = D / 32;         // score MFMAs per tile (32 d each), and V words per lane row
  constexpr int NACC = D / 16;       // accumulator blocks: d = (D / 16) c + e, e < NACC
  constexpr int RB = D * E;          // bytes per token row (256, 128 or 64)
  constexpr bool R8 = RB == 128;
  // scales of a tile: the (block, head) scale, or the lane's four tokens'
  using Sc = typename std::conditional<TOKSC, f32x4_t, float>::type;
  const int lane = threadIdx.x & 63;
  const int wv = WPI > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
  const int j = lane >> 4;
  const int c = lane & 15;
  // wave-uniform: prefix item of a cascade launch
  const bool pre = MODE == kModeCascade && (int)blockIdx.x < cz.items;
  // balanced split: this wave's ranges v = blockIdx.x / Hkv + k * Wh of pw tiles
  TileMap<CH> tm;
  int pw = 1, V = 0, Wh = 1, v = 0, ra = 0, rb = 0;
  if constexpr (BAL) {
    tile_map_init(tm, context_lens, num_rows, max_blocks * BS, bz.cap, lane);
    Wh = gridDim.x / Hkv;
    pw = min(max((tm.total + Wh - 1) / Wh, bz.min_tiles), kBalancedMaxTiles);
    V = (tm.total + pw - 1) / pw;
    v = (int)blockIdx.x / Hkv - Wh;
    if (blockIdx.x == 0) {
      // partials of each sequence: the ranges its tiles meet
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        const int si = 64 * ch + lane;
        const int c = tile_count(tm.len[ch], bz.cap), in = tm.incl[ch];
        if (si < num_rows) ws.counts[si] = c > 0 ? (in - 1) / pw - (in - c) / pw + 1 : 0;
      }
    }
  }
  // one item per wave, except in a balanced split (a loop over pieces)
  for (;;) {
  int s, g, p, cgw, n_piece = 0, piece_t0 = 0, piece_t1 = 0, piece_slot = 0;
  if constexpr (BAL) {
    if (ra >= rb) {
      v += Wh;
      if (v >= V) return;
      ra = v * pw;
      rb = min(tm.total, ra + pw);
    }
    int c, excl;
    tile_find(tm, ra, bz.cap, s, n_piece, c, excl);
    const int lt0 = ra - excl, lt1 = min(c, lt0 + (rb - ra));
    piece_t0 = 16 * lt0;
    piece_t1 = 16 * lt1;
    piece_slot = v - excl / pw;
    ra += lt1 - lt0;
    g = (int)blockIdx.x % Hkv;
    p = 0;
    cgw = 0;
  } else if (pre) {
    mfma_item(blockIdx.x, Hkv, cz.nP, cz.CG, s, g, p, cgw);
  } else if (MODE == kModeCascade) {
    mfma_item(blockIdx.x - cz.items, Hkv, nP, CG, s, g, p, cgw);
  } else if (GROUP) {
    mfma_item(blockIdx.x, Hkv, 1, 1, s, g, p, cgw);  // one column group per item
    p = wv;
  } else {
    mfma_item(blockIdx.x, Hkv, nP, CG, s, g, p, cgw);
  }
  // this wave's tokens: [t_begin, t_end) of a table row of row_blocks entries
  const int32_t* trow = pre ? cz.table : tables + (size_t)s * max_blocks;
  const int row_blocks = pre ? cz.blocks : max_blocks;
  const int Pw = pre ? cz.P : P;
  const int t_begin = BAL ? piece_t0 : (MODE == kModeCascade && !pre ? cz.t0 : 0) + p * Pw;
  // partial slot of this wave's partition, of nPw per row
  const int slot = BAL ? piece_slot : MODE == kModeCascade ? (pre ? p : cz.nP + p) : p;
  const int nPw = MODE == kModeCascade ? cz.nPw : GROUP ? 1 : nP;
  // The partition's table entries, two per lane (a partition spans at most
  // 128 blocks, which the host guarantees): entry i of the partition is
  // lane i of tbl0 or lane i - 64 of tbl1.  They are read before the
  // context length is known, so the two loads overlap; entries past the
  // sequence's blocks (inside the table row) are read and never used.
  const int tbl_base = t_begin / BS;
  const int tbl0 = (tbl_base + lane < row_blocks) ? trow[tbl_base + lane] : -1;
  const int tbl1 = (tbl_base + 64 + lane < row_blocks) ? trow[tbl_base + 64 + lane] : -1;
  // a length past the table row is a caller error; never read beyond the row
  const int n = pre ? cz.blocks * BS : BAL ? n_piece : min(context_lens[s], max_blocks * BS);
  // (a grouped wave past the plan's nP partitions attends to nothing, as
  // no wave would in the other modes)
  const int t_end = GROUP && p >= nP ? t_begin : min(n, BAL ? piece_t1 : t_begin + Pw);
  // this lane's column in each group u: output / partial row orow[u],
  // visible tokens < lim[u] (MQ: several rows per sequence, qsl given)
  bool head_ok[NCG];
  size_t orow[NCG];
  int lim[NCG];
#pragma unroll
  for (int u = 0; u < NCG; ++u) {
    int h, qrow;
    if constexpr (MQ) {
      // without row offsets (more than 16 query heads per kv head): one
      // query row per sequence, row s
      const int q0 = qsl ? qsl[s] : s, L = qsl ? qsl[s + 1] - q0 : 1;
      const int col = 16 * (cgw * NCG + u) + c, i = col / G;
      // rows outside [0, num_rows) (offsets not matching num_queries, a
      // caller error) are neither read nor written
      head_ok[u] = i < L && q0 + i >= 0 && q0 + i < num_rows;
      h = g * G + col % G;
      qrow = q0 + i;
      lim[u] = head_ok[u] ? max(0, min(t_end, n - L + i + 1)) : 0;
      if (u == 0 && 16 * cgw * NCG >= G * L) return;  // no column of these groups exists
    } else if (pre) {
      // prefix column col -> (sequence col / G, head col % G), seeing the
      // prefix up to its own length
      const int col = 16 * (cgw * NCG + u) + c, i = col / G;
      head_ok[u] = i < num_rows;
      h = g * G + col % G;
      qrow = head_ok[u] ? i : 0;
      lim[u] = head_ok[u] ? max(0, min(t_end, min(context_lens[i], max_blocks * BS))) : 0;
    } else {
      head_ok[u] = c < G;
      h = g * G + c;
      qrow = s;
      lim[u] = t_end;
    }
    orow[u] = (size_t)qrow * Hq + h;
  }

  // The lowest visible-token limit over this wave's existing columns: a
  // tile entirely below it (and in the pool) needs no mask, and its scores
  // are all finite.
  int lim_lo = t_end;
  if (MQ || pre) {  // wave-uniform; every other item's columns all see up to t_end
    int lo = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < NCG; ++u) lo = min(lo, head_ok[u] ? lim[u] : 0x7fffffff);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) lo = min(lo, __shfl_xor(lo, d, 64));
    lim_lo = __builtin_amdgcn_readfirstlane(lo);
  }

  if (!GROUP && t_begin >= t_end) {
    // Nothing to attend to.  With one partition the output row is zero;
    // otherwise the partial is marked empty (no weight) for the merge.  (A
    // grouped wave goes on to the combination, which every wave of the
    // workgroup must reach, attending to no tile.)
    if (wv != 0) return;
#pragma unroll
    for (int u = 0; u < NCG; ++u) {
      if (nPw == 1 && head_ok[u]) {
        float4* o = (float4*)(out + orow[u] * D + (D / 4) * j);
#pragma unroll
        for (int k = 0; k < D / 16; ++k) o[k] = float4{0.f, 0.f, 0.f, 0.f};
      } else if (nPw > 1 && head_ok[u] && j == 0) {
        ws.ml[orow[u] * nPw + slot] = float2{kNegInf, 0.f};
      }
    }
    if constexpr (BAL) continue;
    else return;
  }

  // Queries as the B operand: column c of group u, the 8 values of d-chunk
  // (kk*4 + j) [bf16 cache] or (j*4 + kk) [1-byte cache].
  bf16x8_t qf[NCG][KK];
#pragma unroll
  for (int u = 0; u < NCG; ++u)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int chunk = I8 ? j * KK + kk : kk * 4 + j;
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (head_ok[u]) w = *(const u32x4_t*)(q + orow[u] * D + chunk * 8);
      qf[u][kk] = as_bf16x8(w);
    }

  const int tile_begin = t_begin >> 4;
  const int tile_end = (t_end + 15) >> 4;

  constexpr int ROW = D * E;                       // bytes per token row
  constexpr int CPR = ROW / 16;                    // 16 B chunks per row
  const size_t head_stride = (size_t)BS * ROW;     // bytes per (block, kv head)

  // Fused cache write of the newest token (position n - 1): the wave whose
  // partition holds it reads its K row (16 B chunk c per lane c < CPR) and
  // its V row (the lane's sixteenth, as a tile row is read), stores them
  // into the cache slot at the end and attends with them in the tile that
  // holds the position.  A 1-byte cache with per-token scales at head_dim
  // 128 (QW) takes bf16 rows and quantises them first, as
  // pa_quantize_and_cache would: lane c codes d = 8c .. 8c+7 of each row
  // (the same in every 16-lane row), and the new token's scales stand in
  // for the ones in its slot.  The host rejects the other 1-byte forms.
  // (never with several query rows: the host rejects a fused write there)
  constexpr bool QW = I8 && TOKSC && D == 128 && !MQ;
  const int tnew = n - 1;
  const bool owns_new = (!I8 || QW) && !pre && new_k != nullptr && tnew >= cz.write_from && tnew >= t_begin &&
                        tnew < t_end && (TS == 1 || ((tnew >> 4) - (t_begin >> 4)) % TS == wv);  // wave-uniform
  u32x4_t nk = {0u, 0u, 0u, 0u}, nv = {0u, 0u, 0u, 0u};
  float nks = 1.f, nvs = 1.f;
  if (owns_new) {
    if constexpr (QW) {
      const size_t src = ((size_t)s * Hkv + g) * (D * 2);  // bf16 rows
      const u32x2_t kc = quant_row8<KV == kKvFp8>(*(const u32x4_t*)(new_k + src + (size_t)c * 16), nks);
      const u32x2_t vc = quant_row8<KV == kKvFp8>(*(const u32x4_t*)(new_v + src + (size_t)c * 16), nvs);
      // a K chunk of the LDS tile is 16 codes: lane 2m holds chunk m, its
      // own 8 codes then lane 2m + 1's
      nk = u32x4_t{kc[0], kc[1], (unsigned)__shfl_xor((int)kc[0], 1, 64), (unsigned)__shfl_xor((int)kc[1], 1, 64)};
      nv = u32x4_t{vc[0], vc[1], 0u, 0u};
    } else {
      const size_t src = ((size_t)s * Hkv + g) * ROW;
      if (c < CPR) nk = *(const u32x4_t*)(new_k + src + (size_t)c * 16);
      if constexpr (R8) {
        const u32x2_t w = *(const u32x2_t*)(new_v + src + (size_t)c * 8);
        nv = u32x4_t{w[0], w[1], 0u, 0u};
      } else {
        nv = *(const u32x4_t*)(new_v + src + (size_t)c * 16);
      }
    }
  }
  // K goes through a per-wave LDS tile of 16 rows of 16 B chunks (16 per
  // row of 256 bytes, 8 of 128).  Chunk ch of row r sits at position
  // ch ^ (r mod chunks-per-row), so the row-wise writes and the MFMA-layout
  // reads (16 rows, one chunk each) spread over the banks.
  // With several waves per item the same LDS later holds the waves'
  // (m, l, acc) for their combination.
  constexpr int KT_BYTES = WPI * 16 * CPR * 16;
  constexpr int ACC_BYTES = (WPI - 1) * NCG * NACC * 64 * 16;
  constexpr int CMB_BYTES = WPI > 1 ? ACC_BYTES + WPI * NCG * 2 * 64 * 4 : 0;
  __shared__ __attribute__((aligned(16))) char smem[KT_BYTES > CMB_BYTES ? KT_BYTES : CMB_BYTES];
  u32x4_t* ktile = (u32x4_t*)smem + wv * 16 * CPR;
  unsigned koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    koff[i] = lane * 16 + i * 1024;
    voff[i] = (4 * j + i) * ROW + c * (ROW / 16);
  }
  int kw[4], kr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (RB == 64) {
      const int r = lane >> 2, ch = lane & 3;  // the one load of this lane
      kw[i] = r * 4 + (ch ^ (r & 3));
      kr[i] = c * 4 + (j ^ (c & 3));           // read: row c, chunk j (the lane's 16 d, converted)
    } else if (R8) {
      const int r = 8 * (i & 1) + (lane >> 3), ch = lane & 7;  // load i (< 2) of this lane
      kw[i] = r * 8 + (ch ^ (r & 7));
      // read: row c, chunk 2j + (i & 1) of 1-byte codes (the lane's 32 d,
      // converted), chunk (i & 1) * 4 + j of bf16 at head_dim 64
      const int rc = I8 ? 2 * j + (i & 1) : (i & 1) * 4 + j;
      kr[i] = c * 8 + (rc ^ (c & 7));
    } else {
      kw[i] = (4 * i + j) * 16 + (c ^ (4 * i + j));  // write slot of load i
      kr[i] = c * 16 + ((i * 4 + j) ^ c);            // read slot of d-chunk (i*4 + j), row c
    }
  }
  // per-(block, head) scales: NB * Hkv floats (< 2^30 entries: the pool fits one GPU)
  const __amdgpu_buffer_rsrc_t rks = tile_rsrc((const char*)k_scales, NB * Hkv * 4);
  const __amdgpu_buffer_rsrc_t rvs = tile_rsrc((const char*)v_scales, NB * Hkv * 4);
  auto tile_ptrs = [&](int ti, const char*& kb, const char*& vb, bool& ok, Sc& ks, Sc& vs) {
    const int e = (ti * 16) / BS - tbl_base;
    int b = e < 64 ? __builtin_amdgcn_readlane(tbl0, e) : __builtin_amdgcn_readlane(tbl1, e - 64);
    ok = b >= 0 && b < NB;
    if (!ok) b = 0;
    const size_t off = ((size_t)b * Hkv + g) * head_stride + (size_t)((ti * 16) % BS) * ROW;
    kb = k_cache + off;
    vb = v_cache + off;
    if constexpr (TOKSC) {
      // tokens 4j .. 4j+3 of the tile: 16 aligned bytes of the scale row
      const size_t si = ((size_t)b * Hkv + g) * BS + (size_t)((ti * 16) % BS) + 4 * j;
      ks = *(const f32x4_t*)(k_scales + si);
      vs = *(const f32x4_t*)(v_scales + si);
    } else if (I8) {
      // Vector-memory loads, not scalar ones: a scalar load shares the
      // LDS wait counter, so the current tile's wait for its K rows in LDS
      // would also wait for the next tile's scales to arrive from memory.
      const unsigned so = (unsigned)(b * Hkv + g) * 4u;
      ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rks, so, 0, 0));
      vs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rvs, so, 0, 0));
    }
  };

  f32x4_t acc[NCG][NACC];
  float m_run[NCG], l_run[NCG];
#pragma unroll
  for (int u = 0; u < NCG; ++u) {
#pragma unroll
    for (int e = 0; e < NACC; ++e) acc[u][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[u] = kNegInf;
    l_run[u] = 0.f;
  }

  // FULL: every token of the tile is in the pool and visible to every
  // existing column (no mask; the scores, and so the reference, are finite).
  auto compute = [&](auto full_tag, MfmaTile<RB>& T, int ti, bool ok, const Sc& ks_in, const Sc& vs_in) {
    constexpr bool FULL = decltype(full_tag)::value;
    const bool new_tile = owns_new && ti == (tnew >> 4);  // wave-uniform
    const int rnew = tnew & 15;
    Sc ks = ks_in, vs = vs_in;
#pragma unroll
    for (int i = 0; i < RB / 64; ++i) ktile[kw[i]] = T.k[i];
    if (!I8 && new_tile) {
      if (j == 0 && c < CPR) ktile[rnew * CPR + (c ^ (rnew & (CPR - 1)))] = nk;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * j + i == rnew) T.v[i] = nv;
    }
    if constexpr (QW) {
      if (new_tile) {
        if (j == 0 && (c & 1) == 0) ktile[rnew * CPR + ((c >> 1) ^ (rnew & (CPR - 1)))] = nk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (4 * j + i == rnew) {
            T.v[i] = nv;
            ks[i] = nks;
            vs[i] = nvs;
          }
        }
      }
    }
    // ---- scores, one MFMA chain per column group over the same K operands
    bf16x8_t ka[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (I8) {
        // lane holds d = (D / 4) j .. of row c: at head_dim 128 chunk 2j (kk 0, 1)
        // and 2j+1 (kk 2, 3), at 64 chunk j (kk 0, 1)
        const u32x4_t chunk = ktile[kr[kk >> 1]];
        const unsigned w0 = chunk[(kk & 1) * 2], w1 = chunk[(kk & 1) * 2 + 1];
        const u32x2_t lo = codes_to_bf16x4<KV>(w0), hi = codes_to_bf16x4<KV>(w1);
        ka[kk] = as_bf16x8(u32x4_t{lo[0], lo[1], hi[0], hi[1]});
      } else {
        ka[kk] = as_bf16x8(ktile[kr[kk]]);
      }
    }
    const int tok0 = ti * 16 + 4 * j;
    i16x4_t Phi[NCG], Plo[NCG];
#pragma unroll
    for (int u = 0; u < NCG; ++u) {
      f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qf[u][kk], sc, 0, 0, 0);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float xs = qk_log2;
        if constexpr (TOKSC) xs *= ks[r];
        else if (I8) xs *= ks;
        x[r] = (FULL || (ok && tok0 + r < (MODE != kModeDecode ? lim[u] : t_end))) ? sc[r] * xs : kNegInf;
      }
      // ---- lazy rescale of the running reference.  A column's maximum
      // exceeds its reference (the same on the column's four rows) exactly
      // when one of its lanes' own maxima does, so the cross-row maximum is
      // formed only in the rare branch that moves the reference.
      const float xloc = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      if (__any(xloc > m_run[u] + kRescaleThreshold)) {
        const float mloc = xor_max_rows(xloc);
        const bool need = mloc > m_run[u] + kRescaleThreshold;
        const float m_new = need ? mloc : m_run[u];
        const float alpha = need ? fast_exp2(m_run[u] - m_new) : 1.f;
#pragma unroll
        for (int e = 0; e < NACC; ++e) acc[u][e] *= alpha;
        l_run[u] *= alpha;
        m_run[u] = m_new;
      }
      float pw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pw[r] = (FULL || x[r] != kNegInf) ? fast_exp2(x[r] - m_run[u]) : 0.f;
      l_run[u] += (pw[0] + pw[1]) + (pw[2] + pw[3]);
      // (a masked token's V scale may be NaN: its weight stays zero)
      if constexpr (TOKSC) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pw[r] = (FULL || x[r] != kNegInf) ? pw[r] * vs[r] : 0.f;
      } else if (I8) {
#pragma unroll
        for (int r = 0; r < 4; ++r) pw[r] = (FULL || x[r] != kNegInf) ? pw[r] * vs : 0.f;
      }
      // ---- P as bf16 hi + lo, B operand of the P.V MFMA
      float lo[4];
      unsigned hi01 = pack_bf16x2(pw[0], pw[1]), hi23 = pack_bf16x2(pw[2], pw[3]);
      lo[0] = pw[0] - bf16_lo(hi01);
      lo[1] = pw[1] - bf16_hi(hi01);
      lo[2] = pw[2] - bf16_lo(hi23);
      lo[3] = pw[3] - bf16_hi(hi23);
      Phi[u] = as_i16x4(hi01, hi23);
      Plo[u] = as_i16x4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]));
    }
    // ---- V^T operands: rows 4j+i of this lane; rows past the context are
    // zeroed (they may hold NaN and would poison 0 * NaN in the MFMA)
    const bool partial = !FULL && (!ok || ti * 16 + 15 >= t_end);  // wave-uniform
    if (partial) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool keep = ok && tok0 + i < t_end;
#pragma unroll
        for (int w = 0; w < 4; ++w) T.v[i][w] = keep ? T.v[i][w] : 0u;
      }
    }
    unsigned vw[4][KK];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (I8) {
        // 4 codes -> 2 words of bf16 pairs, per code word of the lane's row piece
#pragma unroll
        for (int w2 = 0; w2 < KK / 2; ++w2) {
          const u32x2_t a = codes_to_bf16x4<KV>(T.v[i][w2]);
          vw[i][2 * w2] = a[0];
          vw[i][2 * w2 + 1] = a[1];
        }
      } else {
#pragma unroll
        for (int w = 0; w < KK; ++w) vw[i][w] = T.v[i][w];
      }
    }
#pragma unroll
    for (int w = 0; w < KK; ++w) {
      // word w holds d = (D / 16) c + 2w (low half) and + 2w + 1 (high half)
      const unsigned e01 = __builtin_amdgcn_perm(vw[1][w], vw[0][w], 0x05040100u);
      const unsigned e23 = __builtin_amdgcn_perm(vw[3][w], vw[2][w], 0x05040100u);
      const unsigned o01 = __builtin_amdgcn_perm(vw[1][w], vw[0][w], 0x07060302u);
      const unsigned o23 = __builtin_amdgcn_perm(vw[3][w], vw[2][w], 0x07060302u);
      if constexpr (NCG == 2) {
        // One 32-deep product per (parity, group) instead of two 16-deep
        // ones (which take as long each): K index 8j + e is token 4j + e of
        // the hi weights for e < 4 and of the lo weights for e >= 4, so the
        // V^T operand is this lane's four tokens twice and the weight
        // operand its hi then lo parts.  (The copies cost 16 moves a tile:
        // worth it with two column groups, not with one.)
        const bf16x8_t ae = as_bf16x8(u32x4_t{e01, e23, e01, e23});
        const bf16x8_t ao = as_bf16x8(u32x4_t{o01, o23, o01, o23});
#pragma unroll
        for (int u = 0; u < NCG; ++u) {
          const bf16x8_t pb = as_bf16x8(u32x4_t{__builtin_bit_cast(u32x2_t, Phi[u])[0], __builtin_bit_cast(u32x2_t, Phi[u])[1],
                                                __builtin_bit_cast(u32x2_t, Plo[u])[0], __builtin_bit_cast(u32x2_t, Plo[u])[1]});
          f32x4_t* au = acc[u];
          au[2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, pb, au[2 * w], 0, 0, 0);
          au[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, pb, au[2 * w + 1], 0, 0, 0);
        }
      } else {
        const i16x4_t a_even = as_i16x4(e01, e23);
        const i16x4_t a_odd = as_i16x4(o01, o23);
#pragma unroll
        for (int u = 0; u < NCG; ++u) {
          f32x4_t* au = acc[u];
          au[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_even, Phi[u], au[2 * w], 0, 0, 0);
          au[2 * w] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_even, Plo[u], au[2 * w], 0, 0, 0);
          au[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_odd, Phi[u], au[2 * w + 1], 0, 0, 0);
          au[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_odd, Plo[u], au[2 * w + 1], 0, 0, 0);
        }
      }
    }
  };

  // Software pipeline: the next tile's loads are in flight while the
  // current one is computed.  The last prefetch re-reads the final tile
  // (always in bounds) so every iteration issues the same loads.  The
  // tiles below lim_lo (visible to every existing column) run first with
  // the mask-free tile body, the rest with the masked one, as two loops so
  // that the two bodies are never live together; a fully visible tile
  // whose block id is outside the pool is skipped (it contributes nothing,
  // as the masked body would make it).
  MfmaTile<RB> A, B;
  const char *kA, *vA, *kB, *vB;
  bool okA, okB;
  Sc ksA{}, vsA{}, ksB{}, vsB{};
  auto run_tiles = [&](auto full_tag, auto aux_tag, int ti, int tend) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr int AUX = decltype(aux_tag)::value;
    if (ti >= tend) return;
    tile_ptrs(ti, kA, vA, okA, ksA, vsA);
    mfma_load_tile<RB, AUX>(A, kA, vA, koff, voff);
    while (true) {
      tile_ptrs(ti + TS < tend ? ti + TS : ti, kB, vB, okB, ksB, vsB);
      mfma_load_tile<RB, AUX>(B, kB, vB, koff, voff);
      if (!FULL || okA) compute(full_tag, A, ti, okA, ksA, vsA);
      if ((ti += TS) >= tend) break;
      tile_ptrs(ti + TS < tend ? ti + TS : ti, kA, vA, okA, ksA, vsA);
      mfma_load_tile<RB, AUX>(A, kA, vA, koff, voff);
      if (!FULL || okB) compute(full_tag, B, ti, okB, ksB, vsB);
      if ((ti += TS) >= tend) break;
    }
  };
  // cascade wave wv: tiles tile_begin + wv, + TS, ...; otherwise every tile
  // of the wave's partition.  Tiles below full_end are fully visible.  The
  // split costs the second loop an unoverlapped first load, so a wave takes
  // it only with at least 16 fully visible tiles.
  const int full_end = min(tile_end, max(lim_lo, 0) >> 4);
  int ti = tile_begin + (TS > 1 ? wv : 0);
  // A prefix item's tiles are read again by the other column groups of its
  // kv head: normal loads keep them in L2; every other tile is streamed.
  auto run = [&](auto full_tag, int a, int b) {
    if (MODE == kModeCascade && pre)  // wave-uniform
      run_tiles(full_tag, std::integral_constant<int, 0>{}, a, b);
    else
      run_tiles(full_tag, std::integral_constant<int, 2>{}, a, b);
  };
  if (full_end - ti >= 16 * TS) {
    run(std::true_type{}, ti, full_end);
    ti += (full_end - ti + TS - 1) / TS * TS;
  }
  run(std::false_type{}, ti, tile_end);

  if (owns_new && j == 0) {
    const int e = tnew / BS - tbl_base;
    const int b = e < 64 ? __builtin_amdgcn_readlane(tbl0, e) : __builtin_amdgcn_readlane(tbl1, e - 64);
    if (b >= 0 && b < NB) {
      const size_t dst = ((size_t)b * Hkv + g) * head_stride + (size_t)(tnew % BS) * ROW;
      if constexpr (QW) {
        *(u32x2_t*)(k_cache + dst + (size_t)c * 8) = u32x2_t{nk[0], nk[1]};
        *(u32x2_t*)(v_cache + dst + (size_t)c * 8) = u32x2_t{nv[0], nv[1]};
        if (c == 0) {
          const size_t si = ((size_t)b * Hkv + g) * BS + (size_t)(tnew % BS);
          k_scales[si] = nks;
          v_scales[si] = nvs;
        }
      } else {
        if (c < CPR) *(u32x4_t*)(k_cache + dst + (size_t)c * 16) = nk;
        if constexpr (R8) *(u32x2_t*)(v_cache + dst + (size_t)c * 8) = u32x2_t{nv[0], nv[1]};
        else *(u32x4_t*)(v_cache + dst + (size_t)c * 16) = nv;
      }
    }
  }

  if constexpr (WPI > 1) {
    // Combine the item's waves lane by lane in wave order: each holds its
    // own reference m (-inf: no weight), weight sum l and acc for the same
    // (column, d) slots; wave 0 continues with the combination.
    f32x4_t(*s_acc)[NCG][NACC][64] = (f32x4_t(*)[NCG][NACC][64])smem;
    float(*s_ml)[NCG][2][64] = (float(*)[NCG][2][64])(smem + ACC_BYTES);
    __syncthreads();  // every wave is done with its K tile
#pragma unroll
    for (int u = 0; u < NCG; ++u) {
      s_ml[wv][u][0][lane] = m_run[u];
      s_ml[wv][u][1][lane] = l_run[u];
      if (wv > 0) {
#pragma unroll
        for (int e = 0; e < NACC; ++e) s_acc[wv - 1][u][e][lane] = acc[u][e];
      }
    }
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int u = 0; u < NCG; ++u) {
      float M = m_run[u];
#pragma unroll
      for (int w = 1; w < WPI; ++w) M = fmaxf(M, s_ml[w][u][0][lane]);
      if (M != kNegInf) {
        float f = m_run[u] == kNegInf ? 0.f : fast_exp2(m_run[u] - M);
        l_run[u] *= f;
#pragma unroll
        for (int e = 0; e < NACC; ++e) acc[u][e] *= f;
#pragma unroll
        for (int w = 1; w < WPI; ++w) {
          const float mw = s_ml[w][u][0][lane];
          f = mw == kNegInf ? 0.f : fast_exp2(mw - M);
          l_run[u] = fmaf(f, s_ml[w][u][1][lane], l_run[u]);
#pragma unroll
          for (int e = 0; e < NACC; ++e) acc[u][e] += f * s_acc[w - 1][u][e][lane];
        }
      }
      m_run[u] = M;
    }
  }

  // lane holds d = (D / 4) j + NACC r + e in acc[u][e][r]
#pragma unroll
  for (int u = 0; u < NCG; ++u) {
    const float l_tot = xor_sum_rows(l_run[u]);
    const f32x4_t* a = acc[u];
    if (!head_ok[u]) continue;
    const size_t row_id = orow[u] * nPw + slot;
    const float inv = nPw == 1 ? (l_tot > 0.f ? 1.f / l_tot : 0.f) : 1.f;
    float* o = nPw == 1 ? out + orow[u] * D + (D / 4) * j : ws.acc + row_id * D + (D / 4) * j;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int h = 0; h < NACC / 4; ++h)
        *(float4*)(o + NACC * r + 4 * h) =
            float4{a[4 * h][r] * inv, a[4 * h + 1][r] * inv, a[4 * h + 2][r] * inv, a[4 * h + 3][r] * inv};
    if (nPw > 1 && j == 0) ws.ml[row_id] = float2{m_run[u], l_tot};
  }
  if constexpr (!BAL) return;
  }  // piece loop
}

// ===========================================================================
// Several query rows per sequence with many column groups (long prefill
// chunks): the column-group waves of one (sequence, kv head, partition)
// share its K/V tiles.  A workgroup of W waves loads each 16-token tile
// once -- a sixteenth of a row per thread (8 bf16, or 8 codes of a 1-byte
// cache converted to bf16 by the loader), K in the first 256 threads and V
// in the next 256 -- into an LDS ring of two stages of two tiles, and every
// wave computes its NCG column groups from LDS; one barrier per stage.
// Used with one column group per wave and 16 waves (115-119 VGPRs, 4 waves
// per SIMD): on a 64-row chunk of the 70B-shaped layer 490-501 TFLOP/s,
// against 449 with two column groups per wave in 8-wave workgroups and
// 347-349 for the per-wave kernel.
// Each loader keeps the next stage's chunks in flight in registers (the
// loads past the partition re-read its last tile, so every iteration waits
// for the same number of loads).  head_dim 128; bf16, int8 or E4M3 caches.
//
// Without it every column-group wave reads every tile itself (from L2 after
// the first): a 64-row chunk with 8 query heads per kv head has 32 column
// groups, 16 waves, and is bound by those re-reads, not by its arithmetic
// (the same speed with the softmax, half of the P.V products or the score
// products taken out).
// ===========================================================================
//
// KV: bf16 cache, or 1-byte codes (kKvI8 / kKvFp8) with fp32 scales per
// (block, kv head) or, TOKSC, per token: the loaders convert the codes to
// bf16 into the same LDS layout and stage each row's scales beside the
// tile; the scores and the weights are scaled as in decode_mfma_kernel.
template <int KV, int BS, bool TOKSC, int NCG, int W>
__global__ __launch_bounds__(64 * W) void shared_tile_mq_kernel(
    float* __restrict__ out, SplitK ws, const unsigned short* __restrict__ q, const char* __restrict__ k_cache,
    const char* __restrict__ v_cache, const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ context_lens, int Hq, int Hkv, int G, int NB, float qk_log2, int P, int nP,
    const int32_t* __restrict__ qsl, int CGW, int WGI, int num_rows) {
  constexpr int D = 128;
  constexpr bool I8 = KV != kKvBf16;
  constexpr int ROW = I8 ? D : D * 2;  // bytes per token row in the cache
  constexpr int CPR = 16;              // 16-byte bf16 chunks per row in LDS
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane >> 4;
  const int c = lane & 15;
  // item (sequence s, kv head g, partition p, wave group wgi), kv head fastest
  const int g = (int)blockIdx.x % Hkv;
  int rest = (int)blockIdx.x / Hkv;
  const int wgi = rest % WGI;
  rest /= WGI;
  const int p = rest % nP;
  const int s = rest / nP;
  const int cgw = wgi * W + wv;
  // wave-uniform: a wave past the item's last column groups still loads and
  // takes every barrier
  const bool active = cgw < CGW;
  const int32_t* trow = tables + (size_t)s * max_blocks;
  const int t_begin = p * P;
  // the partition's table entries (at most 128 blocks), two per lane
  const int tbl_base = t_begin / BS;
  const int tbl0_ld = (tbl_base + lane < max_blocks) ? trow[tbl_base + lane] : -1;
  const int tbl1_ld = (tbl_base + 64 + lane < max_blocks) ? trow[tbl_base + 64 + lane] : -1;
  const int n = min(context_lens[s], max_blocks * BS);
  const int t_end = min(n, t_begin + P);
  bool head_ok[NCG];
  size_t orow[NCG];
  int lim[NCG];
  {
    const int q0 = qsl[s], L = qsl[s + 1] - q0;
#pragma unroll
    for (int u = 0; u < NCG; ++u) {
      const int col = 16 * (cgw * NCG + u) + c, i = col / G;
      head_ok[u] = active && i < L && q0 + i >= 0 && q0 + i < num_rows;
      lim[u] = head_ok[u] ? max(0, min(t_end, n - L + i + 1)) : 0;
      orow[u] = (size_t)(q0 + i) * Hq + g * G + col % G;
    }
  }
  // the lowest visible-token limit over this wave's existing columns: tiles
  // below it need no token mask
  int lim_lo = 0x7fffffff;
#pragma unroll
  for (int u = 0; u < NCG; ++u) lim_lo = min(lim_lo, head_ok[u] ? lim[u] : 0x7fffffff);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) lim_lo = min(lim_lo, __shfl_xor(lim_lo, d, 64));
  lim_lo = __builtin_amdgcn_readfirstlane(lim_lo);
  if (t_begin >= t_end) {
    // nothing to attend to (the same for every wave of the workgroup)
#pragma unroll
    for (int u = 0; u < NCG; ++u) {
      if (nP == 1 && head_ok[u]) {
        float4* o = (float4*)(out + orow[u] * D + 32 * j);
#pragma unroll
        for (int k = 0; k < 8; ++k) o[k] = float4{0.f, 0.f, 0.f, 0.f};
      } else if (nP > 1 && head_ok[u] && j == 0) {
        ws.ml[orow[u] * nP + p] = float2{kNegInf, 0.f};
      }
    }
    return;
  }
  bf16x8_t qf[NCG][4];
#pragma unroll
  for (int u = 0; u < NCG; ++u)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (head_ok[u]) w = *(const u32x4_t*)(q + orow[u] * D + (kk * 4 + j) * 8);
      settle(w);
      qf[u][kk] = as_bf16x8(w);
    }
  int tbl0 = tbl0_ld, tbl1 = tbl1_ld;
  settle(tbl0);
  settle(tbl1);

  // Two LDS stages of two tiles (A = the stage's first, B = its second).
  // K: per tile, chunk ch of row r at r * 16 + (ch ^ r), so the
  // MFMA-layout reads of 16 rows spread over the banks.  V: the A operands
  // of the P.V products for both tiles at once, kv_v[stage][parity][w * 64 + l]
  // = for lane l = 16 j + c of any wave, the bf16 of d = 8c + 2w + parity
  // at tokens 4j .. 4j+3 of tile A, then of tile B (read by a wave as 1 KiB
  // in lane order: no bank conflicts).
  __shared__ __attribute__((aligned(16))) u32x4_t kv_k[2][2][16 * CPR];
  __shared__ __attribute__((aligned(16))) u32x4_t kv_v[2][2][16 * CPR];
  // 1-byte codes: each row's K and V scale, kv_s[stage][tile][K / V][row]
  __shared__ __attribute__((aligned(16))) float kv_s[2][2][2][16];
  // the first 2 * 16 * CPR threads (whole waves) load: K chunks, then V
  static_assert(W * 64 >= 2 * 16 * CPR, "a workgroup loads a tile in one pass");
  // (taken from the wave's first lane: the compiler then keeps the cache
  // base and the tile addresses in scalar registers)
  const int wave_tid0 = __builtin_amdgcn_readfirstlane(tid);
  const bool loader = wave_tid0 < 2 * 16 * CPR;
  const bool ld_v = wave_tid0 >= 16 * CPR;
  const int ld_r = (tid & (16 * CPR - 1)) >> 4, ld_ch = tid & 15;
  // a V loader's entries after the transpose: d-pair w = ld_r & 3 (its
  // lane's row within the group of four) of chunk ld_ch, tokens 4 (ld_r >> 2) ..
  const int ld_slot = ld_v ? (ld_r & 3) * 64 + (ld_r >> 2) * 16 + ld_ch : ld_r * 16 + (ld_ch ^ ld_r);
  const char* ld_cache = ld_v ? v_cache : k_cache;
  const float* ld_scales = ld_v ? v_scales : k_scales;
  // per-(block, head) scales: NB * Hkv floats (< 2^30 entries: the pool fits one GPU)
  const __amdgpu_buffer_rsrc_t ld_rsc = tile_rsrc((const char*)ld_scales, I8 && !TOKSC ? NB * Hkv * 4 : 0);
  // each loader's sixteenth of a row: 8 bf16 (16 B) or 8 codes (8 B)
  const unsigned ld_off = (unsigned)(ld_r * ROW + ld_ch * (ROW / 16));
  const size_t head_stride = (size_t)BS * ROW;
  auto block_of = [&](int ti, bool& ok) {
    const int e = (ti * 16) / BS - tbl_base;
    int b = e < 64 ? __builtin_amdgcn_readlane(tbl0, e) : __builtin_amdgcn_readlane(tbl1, e - 64);
    ok = b >= 0 && b < NB;
    return ok ? b : 0;
  };
  // a loader's piece of tile ti (raw codes in the low half for 1-byte
  // caches) and, for 1-byte caches, its row's scale
  auto load_chunk = [&](int ti, float& sc) {
    bool ok;
    const int b = block_of(ti, ok);
    const char* tile = ld_cache + ((size_t)b * Hkv + g) * head_stride + (size_t)((ti * 16) % BS) * ROW;
    const __amdgpu_buffer_rsrc_t rs = tile_rsrc(tile, 16 * ROW);  // uniform tile base, per-lane offset
    if constexpr (I8) {
      if constexpr (TOKSC) {
        sc = ld_scales[((size_t)b * Hkv + g) * BS + (size_t)((ti * 16) % BS) + ld_r];
      } else {
        // a vector-memory load, not a scalar one: a scalar load shares the
        // LDS wait counter, so the wave's next LDS reads would wait for it
        sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ld_rsc, (unsigned)(b * Hkv + g) * 4u, 0, 0));
      }
      const u32x2_t w = bld8(rs, ld_off);
      return u32x4_t{w[0], w[1], 0u, 0u};
    } else {
      (void)sc;
      return bld16(rs, ld_off);
    }
  };
  // 8 codes -> the 8 bf16 of the loader's LDS chunk (exact: every int8 and
  // E4M3 value fits bf16)
  auto to_bf16 = [&](u32x4_t R) {
    if constexpr (I8) {
      const u32x2_t a = codes_to_bf16x4<KV>(R[0]), b = codes_to_bf16x4<KV>(R[1]);
      return u32x4_t{a[0], a[1], b[0], b[1]};
    } else {
      return R;
    }
  };
  // A V loader's chunk R of tile ti -> its {even d, odd d} operand halves.
  // Rows past the partition or of a block outside the pool are zeroed
  // first (they may hold NaN, which a zero weight would not cancel in the
  // MFMA).  Then the chunk is transposed with the other three rows of its
  // 4-row group -- lanes l, l^16, l^32, l^48 hold rows 4j .. 4j+3 of the
  // same chunk, word w = the bf16 pair (d 2w, 2w+1) of the lane's row:
  // after a permlane32 swap on bit 1 of the row index and a permlane16 swap
  // on bit 0, the lane of row i holds word i of all four rows -- and the
  // even and odd d of the four tokens are packed.
  auto v_operands = [&](int ti, u32x4_t R) {
    bool ok;
    (void)block_of(min(ti, (t_end - 1) >> 4), ok);  // a tile past the partition: all rows masked
    if (!ok || ti * 16 + 16 > t_end) {  // wave-uniform
      const bool keep = ok && ti * 16 + ld_r < t_end;
#pragma unroll
      for (int w = 0; w < 4; ++w) R[w] = keep ? R[w] : 0u;
    }
#pragma unroll
    for (int w0 = 0; w0 < 2; ++w0) {
      const u32x2_t a = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(R[w0], R[2 + w0], false, false));
      R[w0] = a[0];
      R[2 + w0] = a[1];
    }
#pragma unroll
    for (int a1 = 0; a1 < 2; ++a1) {
      const u32x2_t b = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(R[2 * a1], R[2 * a1 + 1], false, false));
      R[2 * a1] = b[0];
      R[2 * a1 + 1] = b[1];
    }
    return u32x4_t{__builtin_amdgcn_perm(R[1], R[0], 0x05040100u), __builtin_amdgcn_perm(R[3], R[2], 0x05040100u),
                   __builtin_amdgcn_perm(R[1], R[0], 0x07060302u), __builtin_amdgcn_perm(R[3], R[2], 0x07060302u)};
  };
  // store tiles ti (RA, row scale SA) and ti + 1 (RB, SB) into stage st
  auto store_stage = [&](int st, int ti, u32x4_t RA, u32x4_t RB, float SA, float SB) {
    RA = to_bf16(RA);
    RB = to_bf16(RB);
    if (ld_v) {  // wave-uniform
      const u32x4_t a = v_operands(ti, RA), b = v_operands(ti + 1, RB);
      kv_v[st][0][ld_slot] = u32x4_t{a[0], a[1], b[0], b[1]};
      kv_v[st][1][ld_slot] = u32x4_t{a[2], a[3], b[2], b[3]};
    } else {
      kv_k[st][0][ld_slot] = RA;
      kv_k[st][1][ld_slot] = RB;
    }
    if (I8 && ld_ch == 0) {
      if (ld_v) {
        // a masked row's weight is zero; so is its V scale (the scale of a
        // slot past the context may be NaN)
        bool ok;
        (void)block_of(min(ti, (t_end - 1) >> 4), ok);
        SA = ok && ti * 16 + ld_r < t_end ? SA : 0.f;
        (void)block_of(min(ti + 1, (t_end - 1) >> 4), ok);
        SB = ok && ti * 16 + 16 + ld_r < t_end ? SB : 0.f;
      }
      kv_s[st][0][ld_v][ld_r] = SA;
      kv_s[st][1][ld_v][ld_r] = SB;
    }
  };
  int kr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kr[i] = c * 16 + ((i * 4 + j) ^ c);

  f32x4_t acc[NCG][8];
  float m_run[NCG], l_run[NCG];
#pragma unroll
  for (int u = 0; u < NCG; ++u) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // a finite reference below every score: the first finite score moves
    // it (rescaling zeros), and 2^(-inf - reference) = 0 needs no guard
    m_run[u] = kFloorRef;
    l_run[u] = 0.f;
  }

  // Tiles ti and ti + 1 from stage st (a second tile past the partition is
  // all masked, its V rows zero): both score chains, one rescale check,
  // both weight sets, then the P.V products with 32-deep MFMAs whose K index
  // 8j + e is token 4j + e of tile A for e < 4 and token 4j + e - 4 of tile
  // B for e >= 4 -- so each lane's B operand is its own four weights of
  // each tile, P split into bf16 hi and lo parts in two products.  Tiles
  // every existing column sees whole skip the token mask.
  auto compute = [&](int st, int ti) {
    if (!active) return;
    bool okA, okB;
    (void)block_of(ti, okA);
    (void)block_of(min(ti + 1, (t_end - 1) >> 4), okB);
    const bool full = okA && okB && ti * 16 + 31 < lim_lo;  // wave-uniform
    bf16x8_t ka[4], kb[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      ka[kk] = as_bf16x8(kv_k[st][0][kr[kk]]);
      kb[kk] = as_bf16x8(kv_k[st][1][kr[kk]]);
    }
    const int tok0 = ti * 16 + 4 * j;
    bf16x8_t Phi[NCG], Plo[NCG];
#pragma unroll
    for (int u = 0; u < NCG; ++u) {
      f32x4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[kk], qf[u][kk], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[kk], qf[u][kk], sb, 0, 0, 0);
      }
      float x[8];
      if constexpr (I8) {
        // the scores of 1-byte codes times each token's K scale
        const f32x4_t ksa = *(const f32x4_t*)&kv_s[st][0][0][4 * j], ksb = *(const f32x4_t*)&kv_s[st][1][0][4 * j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = sa[r] * (qk_log2 * ksa[r]);
          x[4 + r] = sb[r] * (qk_log2 * ksb[r]);
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = sa[r] * qk_log2;
          x[4 + r] = sb[r] * qk_log2;
        }
      }
      if (!full) {  // wave-uniform
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[r] = (okA && tok0 + r < lim[u]) ? x[r] : kNegInf;
          x[4 + r] = (okB && tok0 + 16 + r < lim[u]) ? x[4 + r] : kNegInf;
        }
      }
      const float xloc = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                               fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      if (__any(xloc > m_run[u] + kRescaleThreshold)) {
        const float mloc = xor_max_rows(xloc);
        const bool need = mloc > m_run[u] + kRescaleThreshold;
        const float m_new = need ? mloc : m_run[u];
        const float alpha = need ? fast_exp2(m_run[u] - m_new) : 1.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u][e] *= alpha;
        l_run[u] *= alpha;
        m_run[u] = m_new;
      }
      float pw[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) pw[r] = fast_exp2(x[r] - m_run[u]);
      l_run[u] += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
      if constexpr (I8) {
        // the weights times each token's V scale
        const f32x4_t vsa = *(const f32x4_t*)&kv_s[st][0][1][4 * j], vsb = *(const f32x4_t*)&kv_s[st][1][1][4 * j];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pw[r] *= vsa[r];
          pw[4 + r] *= vsb[r];
        }
      }
      unsigned hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        hi[k] = pack_bf16x2(pw[2 * k], pw[2 * k + 1]);
        lo[k] = pack_bf16x2(pw[2 * k] - bf16_lo(hi[k]), pw[2 * k + 1] - bf16_hi(hi[k]));
      }
      Phi[u] = as_bf16x8(u32x4_t{hi[0], hi[1], hi[2], hi[3]});
      Plo[u] = as_bf16x8(u32x4_t{lo[0], lo[1], lo[2], lo[3]});
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x8_t ve = as_bf16x8(kv_v[st][0][w * 64 + lane]);
      const bf16x8_t vo = as_bf16x8(kv_v[st][1][w * 64 + lane]);
#pragma unroll
      for (int u = 0; u < NCG; ++u) {
        f32x4_t* au = acc[u];
        au[2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ve, Phi[u], au[2 * w], 0, 0, 0);
        au[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo, Phi[u], au[2 * w + 1], 0, 0, 0);
        au[2 * w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ve, Plo[u], au[2 * w], 0, 0, 0);
        au[2 * w + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo, Plo[u], au[2 * w + 1], 0, 0, 0);
      }
    }
  };

  const int tile_begin = t_begin >> 4;
  const int tile_end = (t_end + 15) >> 4;
  auto clamp_tile = [&](int ti) { return ti < tile_end ? ti : tile_end - 1; };
  // Stage 0 <- tiles tile_begin, + 1; the next stage's two tiles in flight
  // while a stage is computed.  A loader stores a stage right before it
  // loads the next one, so the wait for its chunks (which the compiler
  // makes a wait for every load in flight) never holds back a newer load:
  // each load has a whole stage, two tiles of compute, to arrive.
  u32x4_t RA = {0u, 0u, 0u, 0u}, RB = {0u, 0u, 0u, 0u};
  float SA = 0.f, SB = 0.f;
  if (loader) {  // wave-uniform
    RA = load_chunk(tile_begin, SA);
    RB = load_chunk(clamp_tile(tile_begin + 1), SB);
    store_stage(0, tile_begin, RA, RB, SA, SB);
    RA = load_chunk(clamp_tile(tile_begin + 2), SA);
    RB = load_chunk(clamp_tile(tile_begin + 3), SB);
  }
  __syncthreads();
  for (int ti = tile_begin;;) {
    compute(0, ti);
    if ((ti += 2) >= tile_end) break;
    if (loader) {
      store_stage(1, ti, RA, RB, SA, SB);  // stage 1 was last read before the previous barrier
      RA = load_chunk(clamp_tile(ti + 2), SA);
      RB = load_chunk(clamp_tile(ti + 3), SB);
    }
    __syncthreads();
    compute(1, ti);
    if ((ti += 2) >= tile_end) break;
    if (loader) {
      store_stage(0, ti, RA, RB, SA, SB);
      RA = load_chunk(clamp_tile(ti + 2), SA);
      RB = load_chunk(clamp_tile(ti + 3), SB);
    }
    __syncthreads();
  }

  // lane holds d = 32j + 8r + e in acc[u][e][r]
#pragma unroll
  for (int u = 0; u < NCG; ++u) {
    const float l_tot = xor_sum_rows(l_run[u]);
    const f32x4_t* a = acc[u];
    if (!head_ok[u]) continue;
    if (nP == 1) {
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      float* o = out + orow[u] * D + 32 * j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *(float4*)(o + 8 * r) = float4{a[0][r] * inv, a[1][r] * inv, a[2][r] * inv, a[3][r] * inv};
        *(float4*)(o + 8 * r + 4) = float4{a[4][r] * inv, a[5][r] * inv, a[6][r] * inv, a[7][r] * inv};
      }
    } else {
      const size_t row_id = orow[u] * nP + p;
      float* o = ws.acc + row_id * D + 32 * j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *(float4*)(o + 8 * r) = float4{a[0][r], a[1][r], a[2][r], a[3][r]};
        *(float4*)(o + 8 * r + 4) = float4{a[4][r], a[5][r], a[6][r], a[7][r]};
      }
      if (j == 0) ws.ml[row_id] = float2{m_run[u], l_tot};
    }
  }
}

// ===========================================================================
// Vector-ALU kernel: any supported dtype, head_dim 64 or 128.
//
// Lane l handles token slot tt = l/16 of each group of four tokens and the
// d-chunk c = l%16 (D/16 consecutive elements).  A score is an in-lane
// partial dot product summed over the 16 lanes of the DPP row.  Each of
// the four token slots keeps its own (m, l, acc) per head; the four are
// merged at the end.
// ===========================================================================

template <typename KV, int DC>
struct KvChunk;

template <int DC>
struct KvChunk<float, DC> {
  static __device__ __forceinline__ void load(const char* p, float (&v)[DC]) {
#pragma unroll
    for (int i = 0; i < DC; i += 4) {
      u32x4_t w = ld16(p + 4 * i);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[i + k] = __uint_as_float(w[k]);
    }
  }
};

template <int DC>
struct KvChunk<__bf16, DC> {
  static __device__ __forceinline__ void load(const char* p, float (&v)[DC]) {
    if constexpr (DC == 8) {
      u32x4_t w = ld16(p);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[2 * k] = bf16_lo(w[k]);
        v[2 * k + 1] = bf16_hi(w[k]);
      }
    } else {
      u32x2_t w = ld8(p);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        v[2 * k] = bf16_lo(w[k]);
        v[2 * k + 1] = bf16_hi(w[k]);
      }
    }
  }
};

template <int DC>
struct KvChunk<signed char, DC> {
  static __device__ __forceinline__ void load(const char* p, float (&v)[DC]) {
    if constexpr (DC == 8) {
      u32x2_t w = ld8(p);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        v[k] = i8_at(w[0], k);
        v[4 + k] = i8_at(w[1], k);
      }
    } else {
      unsigned w = ld4(p);
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = i8_at(w, k);
    }
  }
};

// Tag type of E4M3 cache elements (one byte each).
struct E4M3 {
  unsigned char bits;
};

template <int DC>
struct KvChunk<E4M3, DC> {
  static __device__ __forceinline__ void load(const char* p, float (&v)[DC]) {
    if constexpr (DC == 8) {
      u32x2_t w = ld8(p);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
        const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
        v[4 * k] = lo[0];
        v[4 * k + 1] = lo[1];
        v[4 * k + 2] = hi[0];
        v[4 * k + 3] = hi[1];
      }
    } else {
      const unsigned w = ld4(p);
      const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
      const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
      v[0] = lo[0];
      v[1] = lo[1];
      v[2] = hi[0];
      v[3] = hi[1];
    }
  }
};

template <typename QT, int DC>
__device__ __forceinline__ void load_q(const QT* p, float (&v)[DC]) {
  if constexpr (sizeof(QT) == 4) {
#pragma unroll
    for (int i = 0; i < DC; ++i) v[i] = ((const float*)p)[i];
  } else {
    const unsigned short* u = (const unsigned short*)p;
#pragma unroll
    for (int i = 0; i < DC; ++i) v[i] = __uint_as_float((unsigned)u[i] << 16);
  }
}

template <typename QT, typename KV, int D, int BS, int GT>
__global__ __launch_bounds__(64) void decode_valu_kernel(
    float* __restrict__ out, SplitK ws, const QT* __restrict__ q,
    char* __restrict__ k_cache, char* __restrict__ v_cache, const float* __restrict__ k_scales,
    const float* __restrict__ v_scales, const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ context_lens, int Hq, int Hkv, int G, int head_groups, int NB, float qk_log2,
    int P, int nP, const char* __restrict__ new_k, const char* __restrict__ new_v, int tok_scales,
    int prefix_len) {
  constexpr int DC = D / 16;
  constexpr bool I8 = sizeof(KV) == 1;
  constexpr int E = sizeof(KV);
  const int lane = threadIdx.x;
  const int tt = lane >> 4;
  const int c = lane & 15;
  const int p = blockIdx.x % nP;
  int rest = blockIdx.x / nP;
  const int hg = rest % head_groups;
  rest /= head_groups;
  const int g = rest % Hkv;
  const int s = rest / Hkv;
  const int n = min(context_lens[s], max_blocks * BS);
  const int t_begin = p * P;
  const int t_end = min(n, t_begin + P);
  const int h0 = g * G + hg * GT;
  const int nh = min(GT, G - hg * GT);

  if (t_begin >= t_end) {
    // as in the matrix-core kernel: a zero row, or an empty partial
    if (nP == 1 && tt == 0) {
      for (int i = 0; i < nh; ++i) {
        float* o = out + ((size_t)s * Hq + h0 + i) * D + c * DC;
#pragma unroll
        for (int k = 0; k < DC; ++k) o[k] = 0.f;
      }
    } else if (lane < nh) {
      ws.ml[((size_t)s * Hq + h0 + lane) * nP + p] = float2{kNegInf, 0.f};
    }
    return;
  }

  float qv[GT][DC];
#pragma unroll
  for (int i = 0; i < GT; ++i) {
    if (i < nh) {
      load_q<QT, DC>(q + ((size_t)s * Hq + h0 + i) * D + c * DC, qv[i]);
#pragma unroll
      for (int k = 0; k < DC; ++k) qv[i][k] *= qk_log2;
    } else {
#pragma unroll
      for (int k = 0; k < DC; ++k) qv[i][k] = 0.f;
    }
  }

  float m[GT], l[GT], acc[GT][DC];
#pragma unroll
  for (int i = 0; i < GT; ++i) {
    m[i] = kNegInf;
    l[i] = 0.f;
#pragma unroll
    for (int k = 0; k < DC; ++k) acc[i][k] = 0.f;
  }

  const int32_t* trow = tables + (size_t)s * max_blocks;
  const size_t head_stride = (size_t)BS * D * E;
  // Fused cache write of the newest token (position n - 1): lanes holding
  // that position read its K/V chunk from new_k/new_v instead of the cache;
  // the first head group's wave stores it into the slot at the end.  A
  // position inside a shared prefix (tnew < prefix_len) lies in a block
  // other sequences read: it is neither stored nor taken from new_k/new_v.
  const int tnew = n - 1;
  const bool owns_new = !I8 && new_k != nullptr && tnew >= prefix_len && tnew >= t_begin &&
                        tnew < t_end;  // wave-uniform
  const size_t new_off = ((size_t)s * Hkv + g) * D * E + (size_t)c * DC * E;
  for (int t4 = t_begin; t4 < t_end; t4 += 16) {
    // one 16-token tile: four passes of four tokens
    const int lb = t4 / BS;
    int b = trow[lb];
    const bool ok = b >= 0 && b < NB;
    if (!ok) b = 0;
    const size_t off = ((size_t)b * Hkv + g) * head_stride;
    const int row0 = t4 % BS;
    // scale of each of the lane's four tokens: per (block, head) or per token
    float ksr[4], vsr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ksr[r] = vsr[r] = 1.f;
      if (I8) {
        const size_t si = tok_scales ? ((size_t)b * Hkv + g) * BS + row0 + 4 * r + tt : (size_t)b * Hkv + g;
        ksr[r] = k_scales[si];
        vsr[r] = v_scales[si];
      }
    }
    float kv[4][DC], vv[4][DC];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t roff = off + (size_t)(row0 + 4 * r + tt) * D * E + (size_t)c * DC * E;
      const bool from_new = owns_new && t4 + 4 * r + tt == tnew;
      KvChunk<KV, DC>::load(from_new ? new_k + new_off : k_cache + roff, kv[r]);
      KvChunk<KV, DC>::load(from_new ? new_v + new_off : v_cache + roff, vv[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t4 + 4 * r + tt;
      const bool valid = ok && t < t_end;
      float x[GT];
#pragma unroll
      for (int i = 0; i < GT; ++i) {
        float d = 0.f;
#pragma unroll
        for (int k = 0; k < DC; ++k) d = fmaf(qv[i][k], kv[r][k], d);
        d = row_sum16(d);
        x[i] = valid ? d * ksr[r] : kNegInf;
      }
      bool need = false;
#pragma unroll
      for (int i = 0; i < GT; ++i) need |= x[i] > m[i] + kRescaleThreshold;
      if (__any(need)) {
#pragma unroll
        for (int i = 0; i < GT; ++i) {
          const bool up = x[i] > m[i] + kRescaleThreshold;
          const float m_new = up ? x[i] : m[i];
          const float alpha = up ? fast_exp2(m[i] - m_new) : 1.f;
          l[i] *= alpha;
#pragma unroll
          for (int k = 0; k < DC; ++k) acc[i][k] *= alpha;
          m[i] = m_new;
        }
      }
#pragma unroll
      for (int i = 0; i < GT; ++i) {
        const float pw = valid ? fast_exp2(x[i] - m[i]) : 0.f;
        l[i] += pw;
        const float pv = valid ? pw * vsr[r] : 0.f;  // (a masked slot's scale may be NaN)
#pragma unroll
        for (int k = 0; k < DC; ++k) acc[i][k] = fmaf(pv, valid ? vv[r][k] : 0.f, acc[i][k]);
      }
    }
  }

  if (owns_new && hg == 0 && tt == (tnew & 3)) {
    const int32_t b = trow[tnew / BS];
    if (b >= 0 && b < NB) {
      const size_t dst = ((size_t)b * Hkv + g) * head_stride + (size_t)(tnew % BS) * D * E + (size_t)c * DC * E;
#pragma unroll
      for (int k = 0; k < DC * E; k += 4) {
        *(unsigned*)(k_cache + dst + k) = *(const unsigned*)(new_k + new_off + k);
        *(unsigned*)(v_cache + dst + k) = *(const unsigned*)(new_v + new_off + k);
      }
    }
  }

  // merge the four token slots: common reference, then sums across rows
#pragma unroll
  for (int i = 0; i < GT; ++i) {
    const float mt = xor_max_rows(m[i]);
    const float alpha = m[i] == kNegInf ? 0.f : fast_exp2(m[i] - mt);
    l[i] = xor_sum_rows(l[i] * alpha);
#pragma unroll
    for (int k = 0; k < DC; ++k) acc[i][k] = xor_sum_rows(acc[i][k] * alpha);
    m[i] = mt;
  }
  if (tt == 0) {
#pragma unroll
    for (int i = 0; i < GT; ++i) {
      if (i >= nh) break;
      const int h = h0 + i;
      if (nP == 1) {
        const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;
        float* o = out + ((size_t)s * Hq + h) * D + c * DC;
#pragma unroll
        for (int k = 0; k < DC; ++k) o[k] = acc[i][k] * inv;
      } else {
        const size_t row_id = ((size_t)s * Hq + h) * nP + p;
        float* o = ws.acc + row_id * D + c * DC;
#pragma unroll
        for (int k = 0; k < DC; ++k) o[k] = acc[i][k];
        if (c == 0) ws.ml[row_id] = float2{m[i], l[i]};
      }
    }
  }
}

// ===========================================================================
// launchers
// ===========================================================================

static inline SplitK split_k(const pa_decode_args* a, const DecodePlan& p) {
  SplitK w{nullptr, nullptr, nullptr};
  if (p.ws_partitions > 1) {
    const WorkspaceLayout L = workspace_layout(a, p);
    char* base = (char*)a->workspace;
    w.ml = (float2*)(base + L.ml_offset);
    w.acc = (float*)(base + L.acc_offset);
    if (p.balanced) w.counts = (int32_t*)(base + L.counts_offset);
  }
  return w;
}

pa_status launch_decode_mfma(const pa_decode_args* a, const DecodePlan& p, hipStream_t st) {
  const int ncg = p.ncg, cgw = p.cg_waves;
  Cascade cz{nullptr, 0, 0, 0, 0, 1, 0, p.ws_partitions, a->shared_prefix_len};
  size_t pre_items = 0;
  if (p.cascade) {
    pre_items = (size_t)a->num_kv_heads * p.prefix_partitions * p.prefix_cgroups;
    cz.table = a->shared_prefix_table;
    cz.blocks = a->shared_prefix_len / a->block_size;
    cz.nP = p.prefix_partitions;
    cz.P = p.prefix_tokens;
    cz.CG = p.prefix_cgroups;
    cz.t0 = a->shared_prefix_len;
  }
  if (p.shared_tiles) {
    // workgroups of kSharedWaves waves per (sequence, kv head, partition,
    // wave group), one column group per wave
    const int wgi = (cgw + kSharedWaves - 1) / kSharedWaves;
    const size_t wgs = (size_t)a->num_seqs * a->num_kv_heads * p.num_partitions * wgi;
    if (wgs > 0x7fffffffu) return fail(PA_ERR_UNSUPPORTED, "pa_decode: grid too large");
    const SplitK ws = split_k(a, p);
    const float qk = a->scale * kLog2e;
#define PA_SHARED_LAUNCH(KV, BS, TOKSC, NCG, W)                                                                 \
  hipLaunchKernelGGL((shared_tile_mq_kernel<KV, BS, TOKSC, NCG, W>), dim3((unsigned)wgs), dim3(64 * W), 0, st,  \
                     (float*)a->out, ws, (const unsigned short*)a->q, (const char*)a->k_cache,                  \
                     (const char*)a->v_cache, a->k_scales, a->v_scales, a->block_tables, a->max_blocks_per_seq, \
                     a->context_lens,                                                                           \
                     a->num_q_heads, a->num_kv_heads, p.G, a->num_blocks, qk, p.partition_tokens,               \
                     p.num_partitions, a->query_start_loc, cgw, wgi, a->num_queries)
#define PA_SHARED_BS(KV, TOKSC)                                                  \
  if (a->block_size == 16) PA_SHARED_LAUNCH(KV, 16, TOKSC, 1, kSharedWaves);    \
  else PA_SHARED_LAUNCH(KV, 32, TOKSC, 1, kSharedWaves)
    const bool tok = a->kv_scale_mode == PA_SCALE_TOKEN;
    switch (a->kv_dtype) {
      case PA_I8:
        if (tok) { PA_SHARED_BS(kKvI8, true); } else { PA_SHARED_BS(kKvI8, false); }
        break;
      case PA_FP8_E4M3:
        if (tok) { PA_SHARED_BS(kKvFp8, true); } else { PA_SHARED_BS(kKvFp8, false); }
        break;
      default:
        PA_SHARED_BS(kKvBf16, false);
        break;
    }
#undef PA_SHARED_BS
#undef PA_SHARED_LAUNCH
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode (shared-tile kernel) launch");
  }
  // workgroups: one wave each, kCascadeWaves per cascade item, or one
  // group of p.group_waves per (sequence, kv head)
  const size_t items = p.balanced  ? (size_t)a->num_kv_heads * p.balanced_waves
                       : p.grouped ? (size_t)a->num_seqs * a->num_kv_heads
                                   : pre_items + (size_t)a->num_seqs * a->num_kv_heads * p.num_partitions * cgw;
  const Balanced bz{p.balanced_min_tiles, a->max_context_len};
  if (items > 0x7fffffffu) return fail(PA_ERR_UNSUPPORTED, "pa_decode: grid too large");
  cz.items = (int)pre_items;
  const float qk = a->scale * kLog2e;
  const SplitK ws = split_k(a, p);
#define PA_MFMA_LAUNCH1(KV, BS, TOKSC, NCG, MODE, WG)                                                           \
  hipLaunchKernelGGL((decode_mfma_kernel<KV, BS, TOKSC, NCG, MODE, WG, D>), dim3((unsigned)items), dim3(64 * WG), \
                     0, st,                                                                                    \
                     (float*)a->out, ws, (const unsigned short*)a->q, (char*)a->k_cache, (char*)a->v_cache,      \
                     const_cast<float*>(a->k_scales), const_cast<float*>(a->v_scales), a->block_tables,        \
                     a->max_blocks_per_seq, a->context_lens,                                                   \
                     a->num_q_heads, a->num_kv_heads, p.G, a->num_blocks, qk, p.partition_tokens,              \
                     p.num_partitions, (const char*)a->new_key, (const char*)a->new_value,                     \
                     a->query_start_loc, cgw, a->query_start_loc ? a->num_queries : a->num_seqs, cz, bz)
#define PA_MFMA_GROUP(KV, BS, TOKSC, MODE)                                           \
  do {                                                                               \
    if (p.group_waves == 2) PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, MODE, 2);              \
    else if (p.group_waves == 4) PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, MODE, 4);         \
    else PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, MODE, 8);                                 \
  } while (0)
#define PA_MFMA_LAUNCH(KV, BS, TOKSC)                                                \
  do {                                                                               \
    if (p.cascade) PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, kModeCascade, kCascadeWaves);  \
    else if (p.balanced && a->num_seqs > kBalancedMaxSeqs) PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, kModeBalancedWide, 1); \
    else if (p.balanced) PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, kModeBalanced, 1);        \
    else if (p.grouped && !a->query_start_loc) PA_MFMA_GROUP(KV, BS, TOKSC, kModeDecode); \
    else if (p.grouped) PA_MFMA_GROUP(KV, BS, TOKSC, kModeMultiQuery);                \
    else if (!a->query_start_loc && p.cgroups == 1) PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, kModeDecode, 1); \
    else if (ncg == 2) PA_MFMA_LAUNCH1(KV, BS, TOKSC, 2, kModeMultiQuery, 1);        \
    else PA_MFMA_LAUNCH1(KV, BS, TOKSC, 1, kModeMultiQuery, 1);                      \
  } while (0)
#define PA_MFMA_BS(KV, TOKSC)                              \
  if (a->block_size == 16) PA_MFMA_LAUNCH(KV, 16, TOKSC); \
  else PA_MFMA_LAUNCH(KV, 32, TOKSC)
  const bool tok = a->kv_scale_mode == PA_SCALE_TOKEN;
#define PA_MFMA_KV()                                                                 \
  switch (a->kv_dtype) {                                                             \
    case PA_I8:                                                                      \
      if (tok) { PA_MFMA_BS(kKvI8, true); } else { PA_MFMA_BS(kKvI8, false); }       \
      break;                                                                         \
    case PA_FP8_E4M3:                                                                \
      if (tok) { PA_MFMA_BS(kKvFp8, true); } else { PA_MFMA_BS(kKvFp8, false); }     \
      break;                                                                         \
    default:                                                                         \
      PA_MFMA_BS(kKvBf16, false);                                                    \
      break;                                                                         \
  }
  if (a->head_dim == 64) {
    constexpr int D = 64;
    PA_MFMA_KV();
  } else {
    constexpr int D = 128;
    PA_MFMA_KV();
  }
#undef PA_MFMA_KV
#undef PA_MFMA_BS
#undef PA_MFMA_LAUNCH
#undef PA_MFMA_GROUP
#undef PA_MFMA_LAUNCH1
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode (matrix-core kernel) launch");
}

template <typename QT, typename KV, int D, int BS>
static void valu_dispatch_g(const pa_decode_args* a, const DecodePlan& p, hipStream_t st, unsigned items,
                            const SplitK& ws, float qk) {
#define PA_VALU_LAUNCH(GT)                                                                                    \
  hipLaunchKernelGGL((decode_valu_kernel<QT, KV, D, BS, GT>), dim3(items), dim3(64), 0, st, (float*)a->out,  \
                     ws, (const QT*)a->q, (char*)a->k_cache, (char*)a->v_cache, a->k_scales, \
                     a->v_scales, a->block_tables, a->max_blocks_per_seq, a->context_lens, a->num_q_heads,   \
                     a->num_kv_heads, p.G, p.head_groups, a->num_blocks, qk, p.partition_tokens,             \
                     p.num_partitions, (const char*)a->new_key, (const char*)a->new_value,                \
                     a->kv_scale_mode == PA_SCALE_TOKEN ? 1 : 0, a->shared_prefix_len)
  switch (p.heads_per_wave) {
    case 1: PA_VALU_LAUNCH(1); break;
    case 2: PA_VALU_LAUNCH(2); break;
    case 4: PA_VALU_LAUNCH(4); break;
    default: PA_VALU_LAUNCH(8); break;
  }
#undef PA_VALU_LAUNCH
}

template <typename QT, typename KV>
static void valu_dispatch_shape(const pa_decode_args* a, const DecodePlan& p, hipStream_t st, unsigned items,
                                const SplitK& ws, float qk) {
  if (a->head_dim == 64) {
    if (a->block_size == 16) valu_dispatch_g<QT, KV, 64, 16>(a, p, st, items, ws, qk);
    else valu_dispatch_g<QT, KV, 64, 32>(a, p, st, items, ws, qk);
  } else {
    if (a->block_size == 16) valu_dispatch_g<QT, KV, 128, 16>(a, p, st, items, ws, qk);
    else valu_dispatch_g<QT, KV, 128, 32>(a, p, st, items, ws, qk);
  }
}

template <typename QT>
static void valu_dispatch_kv(const pa_decode_args* a, const DecodePlan& p, hipStream_t st, unsigned items,
                             const SplitK& ws, float qk) {
  switch (a->kv_dtype) {
    case PA_F32: valu_dispatch_shape<QT, float>(a, p, st, items, ws, qk); break;
    case PA_BF16: valu_dispatch_shape<QT, __bf16>(a, p, st, items, ws, qk); break;
    case PA_FP8_E4M3: valu_dispatch_shape<QT, E4M3>(a, p, st, items, ws, qk); break;
    default: valu_dispatch_shape<QT, signed char>(a, p, st, items, ws, qk); break;
  }
}

pa_status launch_decode_valu(const pa_decode_args* a, const DecodePlan& p, hipStream_t st) {
  const size_t items = (size_t)a->num_seqs * a->num_kv_heads * p.head_groups * p.num_partitions;
  if (items > 0x7fffffffu) return fail(PA_ERR_UNSUPPORTED, "pa_decode: grid too large");
  const float qk = a->scale * kLog2e;
  const SplitK ws = split_k(a, p);
  if (a->q_dtype == PA_F32) valu_dispatch_kv<float>(a, p, st, (unsigned)items, ws, qk);
  else valu_dispatch_kv<unsigned short>(a, p, st, (unsigned)items, ws, qk);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode (vector-ALU kernel) launch");
}

template <int D>
static void merge_dispatch(const pa_decode_args* a, const DecodePlan& p, hipStream_t st, unsigned rows,
                           const SplitK& ws, int max_tokens) {
#define PA_MERGE_LAUNCH(W)                                                                                  \
  hipLaunchKernelGGL((decode_merge_kernel<D, W>), dim3(rows), dim3(64 * W), 0, st, (float*)a->out, ws,       \
                     a->query_start_loc || p.cascade || p.balanced ? nullptr : a->context_lens, a->num_q_heads, \
                     p.partition_tokens, p.ws_partitions, max_tokens)
  if (p.ws_partitions <= 16) PA_MERGE_LAUNCH(1);
  else if (p.ws_partitions <= 32) PA_MERGE_LAUNCH(2);
  else if (p.ws_partitions <= 64) PA_MERGE_LAUNCH(4);
  else PA_MERGE_LAUNCH(8);
#undef PA_MERGE_LAUNCH
}

// fp32 -> bf16 (round to nearest even), four values per thread
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float4* __restrict__ in, u32x2_t* __restrict__ out,
                                                          size_t n4) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const float4 v = in[i];
  out[i] = u32x2_t{pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
}

pa_status launch_f32_to_bf16(const float* in, void* out, size_t n, hipStream_t st) {
  const size_t n4 = n / 4;
  if (n4 == 0) return PA_OK;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, (const float4*)in,
                     (u32x2_t*)out, n4);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode (bf16 output) launch");
}

pa_status launch_decode_merge(const pa_decode_args* a, const DecodePlan& p, hipStream_t st) {
  const size_t rows = (size_t)p.rows;
  if (rows == 0) return PA_OK;
  const SplitK ws = split_k(a, p);
  const int max_tokens = a->max_blocks_per_seq * a->block_size;
  if (a->head_dim == 64) merge_dispatch<64>(a, p, st, (unsigned)rows, ws, max_tokens);
  else merge_dispatch<128>(a, p, st, (unsigned)rows, ws, max_tokens);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : hip_fail(e, "pa_decode (merge kernel) launch");
}

}  // namespace pa
