// The host half of libpa under AddressSanitizer and UndefinedBehaviorSanitizer
// (built and run by tests/test_sanitizers.py, no GPU): the block pool
// through long random scripts, checked against reference counts kept here;
// the decode planner over a grid of shapes, dtypes, hints and options; and
// the argument checks of every entry point.  No call here reaches a kernel
// launch: each device entry point is given arguments it rejects first.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <random>
#include <vector>

#include "pa.h"

#define CHECK(c)                                                                     \
  do {                                                                               \
    if (!(c)) {                                                                      \
      std::fprintf(stderr, "check failed at %s:%d: %s\n", __FILE__, __LINE__, #c); \
      std::exit(1);                                                                  \
    }                                                                                \
  } while (0)

static void pool_scripts() {
  for (int seed = 0; seed < 40; ++seed) {
    std::mt19937 rng(seed);
    const int NB = 1 + (int)(rng() % 300);
    std::vector<int32_t> order(NB);
    std::iota(order.begin(), order.end(), 0);
    std::shuffle(order.begin(), order.end(), rng);
    pa_pool* p = nullptr;
    CHECK(pa_pool_create(NB, seed % 2 ? order.data() : nullptr, &p) == PA_OK && p);
    std::vector<int32_t> ref(NB, 0);
    for (int step = 0; step < 3000; ++step) {
      const int op = (int)(rng() % 3);
      const int n = (int)(rng() % 9);
      std::vector<int32_t> ids((size_t)n + 1, 0);
      if (op == 0) {
        const int free_now = pa_pool_num_free(p);
        const pa_status s = pa_block_alloc(p, n, ids.data());
        if (n > free_now) {
          CHECK(s == PA_ERR_OOM && pa_pool_num_free(p) == free_now);
        } else {
          CHECK(s == PA_OK);
          for (int i = 0; i < n; ++i) {
            CHECK(ids[i] >= 0 && ids[i] < NB && ref[ids[i]] == 0);
            ref[ids[i]] = 1;
          }
        }
      } else {
        std::vector<int32_t> held;
        for (int id = 0; id < NB; ++id)
          if (ref[id] > 0) held.push_back(id);
        for (int i = 0; i < n; ++i) {
          const unsigned r = rng() % 20;
          if (r < 17 && !held.empty()) ids[i] = held[rng() % held.size()];
          else if (r < 19) ids[i] = (int32_t)(rng() % NB);
          else ids[i] = rng() % 2 ? -1 - (int32_t)(rng() % 5) : NB + (int32_t)(rng() % 5);
        }
        pa_status expect = PA_OK;
        for (int i = 0; i < n; ++i)
          if (ids[i] < 0 || ids[i] >= NB) expect = PA_ERR_INVALID;
        if (expect == PA_OK) {
          std::vector<int32_t> uses(NB, 0);
          for (int i = 0; i < n; ++i) {
            ++uses[ids[i]];
            if (ref[ids[i]] == 0 || (op == 2 && uses[ids[i]] > ref[ids[i]])) expect = PA_ERR_STATE;
          }
        }
        const pa_status s = op == 1 ? pa_block_share(p, n, ids.data()) : pa_block_free(p, n, ids.data());
        CHECK(s == expect);
        if (s == PA_OK)
          for (int i = 0; i < n; ++i) ref[ids[i]] += op == 1 ? 1 : -1;
      }
      if (step % 16 == 0) {
        int nfree = 0;
        for (int id = 0; id < NB; ++id) {
          CHECK(pa_block_refcount(p, id) == ref[id]);
          nfree += ref[id] == 0;
        }
        CHECK(pa_pool_num_free(p) == nfree && pa_pool_num_blocks(p) == NB);
      }
    }
    CHECK(pa_block_refcount(p, -1) == -1 && pa_block_refcount(p, NB) == -1);
    pa_pool_destroy(p);
  }
  pa_pool* p = nullptr;
  CHECK(pa_pool_create(0, nullptr, &p) == PA_ERR_INVALID && p == nullptr);
  const int32_t not_perm[3] = {0, 2, 2};
  CHECK(pa_pool_create(3, not_perm, &p) == PA_ERR_INVALID && p == nullptr);
  CHECK(pa_pool_create(3, nullptr, nullptr) == PA_ERR_INVALID);
  CHECK(pa_block_alloc(nullptr, 1, nullptr) == PA_ERR_INVALID);
  CHECK(pa_pool_num_free(nullptr) == -1 && pa_block_refcount(nullptr, 0) == -1);
  pa_pool_destroy(nullptr);
}

// A stand-in address for device arrays the planner never dereferences.
static void* fake(uintptr_t k) { return reinterpret_cast<void*>(0x100000u * k); }

static void planner_grid() {
  const int shapes[][2] = {{8, 8}, {64, 8}, {32, 8}, {16, 1}, {40, 40}, {17, 1}, {12, 5}};
  const int lens[] = {0, 1, 17, 2048, 8000, 131072};
  const pa_dtype kvs[] = {PA_F32, PA_BF16, PA_I8, PA_FP8_E4M3};
  long calls = 0, ok = 0;
  for (int S : {0, 1, 3, 64, 300})
    for (const auto& hs : shapes)
      for (int D : {64, 128, 96})
        for (int BS : {16, 32, 8})
          for (pa_dtype kv : kvs)
            for (int ml : lens)
              for (int variant = 0; variant < 6; ++variant) {
                pa_decode_args a;
                std::memset(&a, 0, sizeof a);
                a.struct_size = sizeof a;
                a.q_dtype = variant % 2 ? PA_F32 : PA_BF16;
                a.kv_dtype = kv;
                a.out_dtype = PA_F32;
                a.num_seqs = S;
                a.num_q_heads = hs[0];
                a.num_kv_heads = hs[1];
                a.head_dim = D;
                a.block_size = BS;
                a.max_context_len = ml;
                a.max_blocks_per_seq = ml > 0 ? (ml + BS - 1) / BS : 1;
                a.num_blocks = S * a.max_blocks_per_seq + 1;
                a.scale = 0.125f;
                if (kv == PA_I8 || kv == PA_FP8_E4M3) {
                  a.k_scales = (const float*)fake(1);
                  a.v_scales = (const float*)fake(2);
                  a.kv_scale_mode = variant % 3 == 0 ? PA_SCALE_TOKEN : PA_SCALE_BLOCK;
                }
                a.kernel = variant % 3;
                if (variant == 1) a.total_context_len = (int64_t)S * ml / 9;
                if (variant == 2) a.total_context_len = (int64_t)S * ml;
                if (variant == 3) a.partition_tokens = 256;
                if (variant == 4) {
                  a.query_start_loc = (const int32_t*)fake(3);
                  a.max_query_len = 1 + ml % 65;
                  a.num_queries = S * a.max_query_len;
                }
                if (variant == 5 && ml >= 2 * BS) {
                  a.shared_prefix_table = (const int32_t*)fake(4);
                  a.shared_prefix_len = 2 * BS;
                  a.total_context_len = (int64_t)S * ml / 2;
                }
                size_t bytes = 0;
                const pa_status s = pa_decode_workspace_size(&a, &bytes);
                CHECK(s == PA_OK || s == PA_ERR_INVALID || s == PA_ERR_UNSUPPORTED);
                CHECK(s != PA_OK || bytes < ((size_t)1 << 40));
                ++calls;
                if (s == PA_OK) {
                  ++ok;
                  // the same arguments without an output: rejected before any launch
                  if (S > 0) CHECK(pa_decode(&a) == PA_ERR_INVALID && std::strlen(pa_last_error()) > 0);
                }
              }
  std::printf("planner: %ld argument sets, %ld accepted\n", calls, ok);
  CHECK(ok > 1000);
  pa_decode_args a;
  std::memset(&a, 0, sizeof a);
  a.struct_size = sizeof a - 8;
  size_t bytes;
  CHECK(pa_decode_workspace_size(&a, &bytes) == PA_ERR_INVALID);
  CHECK(pa_decode(nullptr) == PA_ERR_INVALID);
}

static void cache_ops_arguments() {
  CHECK(pa_reshape_and_cache(nullptr, nullptr, nullptr, nullptr, PA_BF16, nullptr, 3, 8, 128, 16, 10, nullptr) ==
        PA_ERR_INVALID);
  CHECK(pa_reshape_and_cache(nullptr, nullptr, nullptr, nullptr, PA_BF16, nullptr, 0, 8, 128, 16, 10, nullptr) ==
        PA_OK);
  CHECK(pa_reshape_and_cache(fake(1), fake(2), fake(3), fake(4), PA_I8, (const int64_t*)fake(5), 3, 8, 128, 16, 10,
                             nullptr) == PA_ERR_UNSUPPORTED);
  CHECK(pa_reshape_and_cache(fake(1), fake(2), fake(3), fake(4), PA_BF16, (const int64_t*)fake(5), 3, 8, 96, 16, 10,
                             nullptr) == PA_ERR_INVALID);
  CHECK(pa_copy_blocks(fake(1), fake(2), PA_BF16, nullptr, nullptr, 0, (const int64_t*)fake(3), -1, 8, 128, 16, 10,
                       nullptr) == PA_ERR_INVALID);
  CHECK(pa_copy_blocks(fake(1), fake(2), PA_I8, nullptr, nullptr, 0, (const int64_t*)fake(3), 2, 8, 128, 16, 10,
                       nullptr) == PA_ERR_INVALID);
  CHECK(pa_copy_blocks(nullptr, fake(2), PA_BF16, nullptr, nullptr, 0, (const int64_t*)fake(3), 2, 8, 128, 16, 10,
                       nullptr) == PA_ERR_INVALID);
  CHECK(pa_swap_blocks(fake(1), fake(2), nullptr, nullptr, fake(3), fake(4), nullptr, nullptr, PA_BF16, 0,
                       (const int64_t*)fake(5), -1, 8, 128, 16, 10, 10, nullptr) == PA_ERR_INVALID);
  CHECK(pa_swap_blocks(fake(1), fake(2), (const float*)fake(6), nullptr, fake(3), fake(4), nullptr, nullptr,
                       PA_I8, 0, (const int64_t*)fake(5), 1, 8, 128, 16, 10, 10, nullptr) == PA_ERR_INVALID);
  CHECK(pa_quantize_and_cache(fake(1), fake(2), PA_BF16, fake(3), fake(4), PA_BF16, (float*)fake(5),
                              (float*)fake(6), 0, 1.f, 1.f, (const int64_t*)fake(7), 1, 8, 128, 16, 10,
                              nullptr) == PA_ERR_INVALID);
  CHECK(pa_quantize_and_cache(fake(1), fake(2), PA_BF16, fake(3), fake(4), PA_I8, (float*)fake(5), (float*)fake(6),
                              PA_SCALE_BLOCK, -1.f, 1.f, (const int64_t*)fake(7), 1, 8, 128, 16, 10,
                              nullptr) == PA_ERR_INVALID);
  CHECK(pa_slot_mapping((const int32_t*)fake(1), 4, 2, nullptr, nullptr, nullptr, 2, 16, (int64_t*)fake(2),
                        nullptr) == PA_ERR_INVALID);
  CHECK(pa_slot_mapping((const int32_t*)fake(1), 4, 2, nullptr, nullptr, (const int32_t*)fake(3), 3, 16,
                        (int64_t*)fake(2), nullptr) == PA_ERR_INVALID);
  for (int s = 0; s <= 7; ++s) CHECK(pa_status_string((pa_status)s) != nullptr);
  CHECK(std::strcmp(pa_status_string((pa_status)7), "PA_ERR_UNKNOWN") == 0);
  CHECK(pa_abi_version() == PA_ABI_VERSION);
}

int main() {
  pool_scripts();
  planner_grid();
  cache_ops_arguments();
  std::printf("ok\n");
  return 0;
}
