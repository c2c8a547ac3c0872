// Host-side argument handling of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (the library's host code only, no device code)
// by tests/test_sanitizers.py and run without a GPU: descriptor and stride
// validation over seeded random descriptors (extreme sizes included),
// workspace-size queries of every op, the prefill CSR offsets, the tuning
// options, and every entry point given bad arguments, all of which must
// return a status before anything is launched. Exit status 0 = all passed.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "../../include/kascade.h"

static int failures = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "%s:%d: check failed: %s (%s)\n", __FILE__, __LINE__, #c, \
              kas_last_error());                                              \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

static uint64_t rng = 12345;
static uint64_t next() {
  rng = rng * 6364136223846793005ull + 1442695040888963407ull;
  return rng >> 17;
}
static int64_t pick(const std::vector<int64_t>& v) { return v[next() % v.size()]; }

static kas_desc_t base_desc() {
  kas_desc_t d;
  memset(&d, 0, sizeof(d));
  d.batch = 4; d.n_q_heads = 32; d.n_kv_heads = 8; d.head_dim = 128; d.seq_len = 131072;
  d.topk_pct = 10; d.tile = 32; d.dtype = KAS_DTYPE_BF16;
  return d;
}

int main() {
  // topk rule and CSR offsets
  for (int64_t n = -3; n < 500; ++n)
    for (int pct = -1; pct <= 101; ++pct) {
      const int64_t k = kas_topk_count(n, pct);
      CHECK(k >= 0 && k <= (n > 0 ? n : 0));
    }
  for (int64_t n : {32ll, 64ll, 4096ll, 131072ll, 2097152ll}) {
    kas_desc_t d = base_desc();
    d.seq_len = n;
    std::vector<int64_t> off(n / 32 + 1, -1);
    int64_t total = -1;
    CHECK(kas_prefill_index_offsets(&d, off.data(), &total) == KAS_OK || n > 1000000);
    if (n <= 1000000) CHECK(off.back() == total && off[0] == 0);
  }
  // random descriptors: every query either succeeds or fails with a status
  const std::vector<int64_t> big = {0, 1, 2, 3, 7, 8, 16, 31, 32, 33, 64, 96, 128, 1000, 4096, 65536, 131072,
                                    1 << 20, (1ll << 31) - 1, 1ll << 31, 1ll << 40, -1, -64};
  const std::vector<int64_t> small = {-1, 0, 1, 2, 3, 4, 8, 16, 32, 64, 100, 128, 256, 512};
  int ok = 0;
  for (int it = 0; it < 20000; ++it) {
    // a valid descriptor with one to three fields replaced at random
    kas_desc_t d = base_desc();
    int64_t* st[6] = {&d.q_batch_stride, &d.q_head_stride, &d.q_token_stride,
                      &d.o_batch_stride, &d.o_head_stride, &d.o_token_stride};
    const int nmut = 1 + (int)(next() % 3);
    for (int m = 0; m < nmut; ++m) {
      switch (next() % 16) {
        case 0: d.batch = (int32_t)pick(small); break;
        case 1: d.n_q_heads = (int32_t)pick(small); break;
        case 2: d.n_kv_heads = (int32_t)pick(small); break;
        case 3: d.head_dim = (int32_t)pick({64, 128, 96, 0}); break;
        case 4: d.seq_len = pick(big); break;
        case 5: d.topk_pct = (int32_t)pick({-1, 0, 1, 10, 50, 100, 101}); break;
        case 6: d.tile = (int32_t)pick({32, 16, 0}); break;
        case 7: d.dtype = (int32_t)pick({0, 1, 2, 3, -1}); break;
        case 8: d.softmax_scale = (float)pick({0, 1, -1}); break;
        case 9: d.kv_batch_stride = pick(big); break;
        case 10: d.kv_head_stride = pick(big); break;
        case 11: d.pool_scope = (int32_t)pick({0, 1, 2}); break;
        case 12: d.pool_op = (int32_t)pick({0, 1, -1}); break;
        case 13: d.query_head_map = (int32_t)pick({0, 1, 2}); break;
        default: *st[next() % 6] = pick(big); break;
      }
    }
    for (int op = -1; op <= 6; ++op) {
      size_t bytes = 0;
      const kas_status_t s = kas_workspace_size(&d, op, &bytes);
      CHECK(s >= KAS_OK && s <= KAS_ERR_HIP);
      if (s == KAS_OK) ++ok;
    }
    size_t rb = 0;
    kas_workspace_size_refine(&d, pick(big), &rb);
    int64_t total = 0;
    kas_prefill_index_offsets(&d, nullptr, &total);
  }
  CHECK(ok > 1000);
  // entry points with bad arguments return before any launch
  kas_desc_t d = base_desc();
  d.seq_len = 4096;
  void* fake = (void*)(uintptr_t)(1 << 20);
  void* mis = (void*)(uintptr_t)((1 << 20) + 2);
  size_t need = 0;
  CHECK(kas_workspace_size(&d, KAS_OP_DECODE_ANCHOR, &need) == KAS_OK && need > 0);
  CHECK(kas_decode_anchor(&d, nullptr, fake, fake, (int32_t*)fake, fake, fake, need, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_decode_anchor(&d, mis, fake, fake, (int32_t*)fake, fake, fake, need, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_decode_anchor(&d, fake, fake, fake, (int32_t*)fake, fake, fake, need - 1, nullptr) == KAS_ERR_WORKSPACE_TOO_SMALL);
  CHECK(kas_decode_anchor(&d, fake, fake, fake, (int32_t*)fake, fake, mis, need, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_decode_reuse(&d, fake, fake, fake, nullptr, 8, nullptr, fake, fake, need, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_decode_reuse(&d, fake, fake, fake, (int32_t*)fake, 0, nullptr, fake, fake, need, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_decode_dense(&d, fake, fake, nullptr, fake, fake, need, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_decode_refine(&d, fake, fake, fake, (int32_t*)fake, 8, 1, nullptr, (int32_t*)fake, fake, fake, need,
                          nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_prefill_anchor(&d, fake, fake, fake, nullptr, fake, fake, 1ull << 40, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_prefill_reuse(&d, fake, fake, fake, (int32_t*)fake, 8, nullptr, nullptr, fake, 1ull << 40, nullptr) ==
        KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_prefill_dense(&d, fake, fake, fake, mis, nullptr, 0, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  kas_desc_t ov = d;
  ov.o_token_stride = 64;   // prefill o rows overlap
  CHECK(kas_prefill_dense(&ov, fake, fake, fake, fake, nullptr, 0, nullptr) == KAS_ERR_INVALID_ARGUMENT);
  kas_kv_cache_t c;
  memset(&c, 0, sizeof(c));
  c.block_table = (const int32_t*)fake;
  c.page_size = 24;         // not a power of two
  c.max_pages = 1 << 20;
  c.num_pages = 4;
  CHECK(kas_decode_anchor_kv(&d, &c, fake, fake, fake, (int32_t*)fake, fake, fake, need, nullptr) ==
        KAS_ERR_INVALID_ARGUMENT);
  c.page_size = 16;
  c.max_pages = 2;          // does not cover seq_len
  CHECK(kas_decode_reuse_kv(&d, &c, fake, fake, fake, (int32_t*)fake, 8, nullptr, fake, fake, need, nullptr) ==
        KAS_ERR_INVALID_ARGUMENT);
  // the no-allocation reuse call: checked before any device query
  kas_desc_t nb = base_desc();
  nb.batch = 1024; nb.n_q_heads = 64; nb.seq_len = 64;
  CHECK(kas_decode_reuse_noalloc(&nb, fake, fake, fake, (int32_t*)fake, 8, nullptr, fake, nullptr) ==
        KAS_ERR_UNSUPPORTED);
  CHECK(kas_decode_reuse_noalloc(&d, nullptr, fake, fake, (int32_t*)fake, 8, nullptr, fake, nullptr) ==
        KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_decode_reuse_noalloc(nullptr, fake, fake, fake, (int32_t*)fake, 8, nullptr, fake, nullptr) ==
        KAS_ERR_INVALID_ARGUMENT);
  // options
  int64_t v = 0;
  CHECK(kas_get_option(KAS_OPT_DECODE_SPLIT_ROWS, &v) == KAS_OK && v == -1);
  CHECK(kas_set_option(KAS_OPT_DECODE_SPLIT_ROWS, 15) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_set_option(KAS_OPT_COUNT_, 1) == KAS_ERR_INVALID_ARGUMENT);
  CHECK(kas_set_option(KAS_OPT_PREFILL_POOL_MB, 1) == KAS_OK);
  size_t small_ws = 0, full_ws = 0;
  CHECK(kas_workspace_size(&d, KAS_OP_PREFILL_ANCHOR, &small_ws) == KAS_OK);
  CHECK(kas_set_option(KAS_OPT_PREFILL_POOL_MB, -1) == KAS_OK);
  CHECK(kas_workspace_size(&d, KAS_OP_PREFILL_ANCHOR, &full_ws) == KAS_OK);
  CHECK(small_ws <= full_ws);
  // strings
  char buf[16];
  CHECK(kas_profile_names(buf, sizeof(buf)) == KAS_ERR_INVALID_ARGUMENT);
  std::vector<char> names(4096);
  CHECK(kas_profile_names(names.data(), names.size()) == KAS_OK);
  for (int s = -1; s <= 5; ++s) CHECK(kas_status_string((kas_status_t)s) != nullptr);
  printf("abi driver: %d failure(s), %d successful workspace queries\n", failures, ok);
  return failures ? 1 : 0;
}
