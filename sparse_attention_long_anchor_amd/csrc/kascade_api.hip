// C ABI of the Kascade sparse-attention library (declared in include/kascade.h):
// host-side argument checks, workspace layout, kernel sequencing, optional
// kernel timing. Every launch goes to the caller's stream; nothing here
// allocates device memory or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kascade.h"
#include "kas_internal.hpp"
#include "kas_prefill.hpp"

namespace kas {

// ------------------------------------------------------------------ errors

static thread_local std::string t_last_error;

static kas_status_t fail(kas_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  t_last_error = buf;
  return st;
}

// ------------------------------------------------------------------ timing registry

static const char* const kKernelNames[] = {
    "decode_score", "decode_pool", "select_cand", "select_resolve",
    "select_compact", "select_fused", "decode_attn", "decode_attn_anchor", "decode_combine", "prefill_stats", "prefill_pool",
    "prefill_select", "prefill_attn", "decode_dense", "prefill_dense", "prefill_pool_heads", "decode_page_rows", "decode_refine_map",
    "decode_refine_lens", "prefill_page_copy"};
static_assert(sizeof(kKernelNames) / sizeof(kKernelNames[0]) == K_COUNT_, "one timing name per kernel id");

const char* kernel_name(int id) { return (id >= 0 && id < K_COUNT_) ? kKernelNames[id] : "?"; }

struct Record { int kid; hipEvent_t e0, e1; };
static std::mutex g_prof_mu;
static bool g_prof_on = false;
static std::vector<Record> g_pending;
static std::vector<hipEvent_t> g_free_events;
static double g_total_ms[K_COUNT_];
static int64_t g_launches[K_COUNT_];
static hipEvent_t take_event() {
  if (!g_free_events.empty()) {
    hipEvent_t e = g_free_events.back();
    g_free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void LaunchCtx::begin(int kid) {
  (void)kid;
  e0 = e1 = nullptr;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  hipEvent_t a = take_event();
  hipEvent_t b = a ? take_event() : nullptr;
  if (a && b) {
    e0 = a;
    e1 = b;
  } else if (a) {
    g_free_events.push_back(a);
  }
}

hipError_t LaunchCtx::end(int kid) {
  hipError_t err = hipGetLastError();
  if (e0) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (err == hipSuccess) {
      g_pending.push_back({kid, e0, e1});
    } else {
      g_free_events.push_back(e0);
      g_free_events.push_back(e1);
    }
    e0 = e1 = nullptr;
  }
  return err;
}

static void drain_pending_locked() {
  for (auto& r : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.e1) == hipSuccess && hipEventElapsedTime(&ms, r.e0, r.e1) == hipSuccess) {
      g_total_ms[r.kid] += ms;
      g_launches[r.kid] += 1;
    }
    g_free_events.push_back(r.e0);
    g_free_events.push_back(r.e1);
  }
  g_pending.clear();
}

// ------------------------------------------------------------------ descriptors

struct Shape {
  int B, Hq, Hkv, D, G;
  int64_t N;
  int pct, tile, dtype;
  int scope, op;                    // anchor pooling variant (kas_desc_t.pool_scope / pool_op)
  int qmap;                         // reuse: head_map per query head (kas_desc_t.query_head_map)
  int dense_out;                    // anchor: dense output (kas_desc_t.anchor_dense_output)
  float scale;
  int64_t kv_hs, kv_bs;
  int64_t q_bs, q_hs, q_ts, o_bs, o_hs, o_ts;   // element strides of q and o
  size_t esize;
};

static int64_t topk_count(int64_t n, int32_t pct) {
  if (n <= 0 || pct <= 0) return 0;
  int64_t k = ((int64_t)pct * n + 50) / 100;
  return k > n ? n : k;
}
static int64_t decode_k(int64_t n, int32_t pct) {
  int64_t k = topk_count(n, pct);
  return (k < 1 && n >= 1) ? 1 : k;
}

static kas_status_t check_desc(const kas_desc_t* d, bool prefill, Shape& s) {
  if (!d) return fail(KAS_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->batch < 1 || d->n_kv_heads < 1 || d->n_q_heads < 1)
    return fail(KAS_ERR_INVALID_ARGUMENT, "batch/heads must be >= 1");
  if (d->n_q_heads % d->n_kv_heads)
    return fail(KAS_ERR_INVALID_ARGUMENT, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                d->n_q_heads, d->n_kv_heads);
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(KAS_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(KAS_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", d->head_dim);
  if (d->seq_len < 1 || d->seq_len >= (int64_t(1) << 31))
    return fail(KAS_ERR_INVALID_ARGUMENT, "seq_len must be in [1, 2^31)");
  if (d->topk_pct < 1 || d->topk_pct > 100)
    return fail(KAS_ERR_INVALID_ARGUMENT, "topk_pct must be in [1, 100]");
  if (d->dtype != KAS_DTYPE_F32 && d->dtype != KAS_DTYPE_BF16 && d->dtype != KAS_DTYPE_F16)
    return fail(KAS_ERR_INVALID_ARGUMENT, "unknown dtype %d", d->dtype);
  if (!(d->softmax_scale == d->softmax_scale) || isinf(d->softmax_scale))
    return fail(KAS_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if ((d->pool_scope != 0 && d->pool_scope != 1) || (d->pool_op != 0 && d->pool_op != 1))
    return fail(KAS_ERR_INVALID_ARGUMENT, "pool_scope and pool_op must be 0 or 1");
  if (d->query_head_map != 0 && d->query_head_map != 1)
    return fail(KAS_ERR_INVALID_ARGUMENT, "query_head_map must be 0 or 1");
  if (d->anchor_dense_output != 0 && d->anchor_dense_output != 1)
    return fail(KAS_ERR_INVALID_ARGUMENT, "anchor_dense_output must be 0 or 1");
  if (d->pool_scope == 1 && d->n_q_heads > kMaxPoolHeads)
    return fail(KAS_ERR_UNSUPPORTED, "pooling over all heads supports at most %d query heads", kMaxPoolHeads);
  if (prefill) {
    if (d->dtype == KAS_DTYPE_F32) return fail(KAS_ERR_UNSUPPORTED, "prefill supports bf16 and fp16 only");
    if (d->tile != 32) return fail(KAS_ERR_UNSUPPORTED, "prefill tile must be 32 (got %d)", d->tile);
    if (d->seq_len % 32) return fail(KAS_ERR_UNSUPPORTED, "prefill seq_len must be a multiple of 32");
  }
  s.B = d->batch; s.Hq = d->n_q_heads; s.Hkv = d->n_kv_heads; s.D = d->head_dim; s.G = G;
  s.N = d->seq_len; s.pct = d->topk_pct; s.tile = d->tile; s.dtype = d->dtype;
  s.scope = d->pool_scope; s.op = d->pool_op; s.qmap = d->query_head_map; s.dense_out = d->anchor_dense_output;
  s.scale = d->softmax_scale > 0.f ? d->softmax_scale : (float)(1.0 / sqrt((double)d->head_dim));
  s.esize = d->dtype == KAS_DTYPE_F32 ? 4 : 2;
  s.kv_hs = d->kv_head_stride ? d->kv_head_stride : s.N * s.D;
  s.kv_bs = d->kv_batch_stride ? d->kv_batch_stride : s.Hkv * s.kv_hs;
  if (s.kv_hs < s.N * s.D || s.kv_bs < (s.Hkv - 1) * s.kv_hs + s.N * s.D)
    return fail(KAS_ERR_INVALID_ARGUMENT, "kv strides overlap the [N, D] rows of a head");
  const int64_t vec = 16 / (int64_t)s.esize;
  if (s.kv_hs % vec || s.kv_bs % vec)
    return fail(KAS_ERR_INVALID_ARGUMENT, "kv strides must be multiples of 16 bytes");
  // q and o: [B, Hq, (N,) D] by default; given strides replace the defaults
  const int64_t rows = prefill ? s.N : 1;
  const int64_t dflt[3] = {(int64_t)s.Hq * rows * s.D, rows * s.D, s.D};
  const int64_t qs[3] = {d->q_batch_stride, d->q_head_stride, d->q_token_stride};
  const int64_t os[3] = {d->o_batch_stride, d->o_head_stride, d->o_token_stride};
  int64_t* qdst[3] = {&s.q_bs, &s.q_hs, &s.q_ts};
  int64_t* odst[3] = {&s.o_bs, &s.o_hs, &s.o_ts};
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || os[i] < 0 || qs[i] % vec || os[i] % vec)
      return fail(KAS_ERR_INVALID_ARGUMENT, "q/o strides must be 0 or positive multiples of 16 bytes");
    *qdst[i] = qs[i] ? qs[i] : dflt[i];
    *odst[i] = os[i] ? os[i] : dflt[i];
  }
  // o rows must not overlap: with the dimensions of more than one entry in
  // ascending stride order, each stride must clear the span of the smaller ones
  {
    struct Dim { int64_t stride, size; } dims[3] = {{s.o_bs, s.B}, {s.o_hs, s.Hq}, {s.o_ts, rows}};
    std::sort(dims, dims + 3, [](const Dim& x, const Dim& y) { return x.stride < y.stride; });
    int64_t span = s.D;
    for (const Dim& dm : dims) {
      if (dm.size <= 1) continue;
      if (dm.stride < span) return fail(KAS_ERR_INVALID_ARGUMENT, "o strides make output rows overlap");
      span = dm.stride * (dm.size - 1) + span;
    }
  }
  return KAS_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static kas_status_t check_ptr(const void* p, const char* name) {
  if (!p) return fail(KAS_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(KAS_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", name);
  return KAS_OK;
}

// ------------------------------------------------------------------ workspace plans

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------------------------ tuning options

static std::atomic<int64_t> g_options[KAS_OPT_COUNT_] = {{-1}, {-1}, {-1}, {-1}};

int64_t option_value(int id) {
  return (id >= 0 && id < KAS_OPT_COUNT_) ? g_options[id].load(std::memory_order_relaxed) : -1;
}

// Compute units of the current device (cached per device; 256 on MI355X).
// Calls from several threads may query the same device at once: the cache
// entries are atomics, and concurrent first queries store the same value.
static int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Rows of the index set per decode attention workgroup. The gather is bound
// by bytes in flight, and a workgroup keeps its waves' next blocks in flight,
// so one wave of workgroups covering every compute unit once is enough:
// splits per (b, g) = CUs / (B * Hkv), at most kMaxSplitRows rows each.
static int decode_split_rows(int64_t units, int64_t kk) {
  int r = (int)option_value(KAS_OPT_DECODE_SPLIT_ROWS);
  if (r <= 0) {
    const int64_t splits = std::max<int64_t>(1, device_cus() / std::max<int64_t>(1, units));
    int64_t per = (kk + splits - 1) / splits;
    per = (per + 63) / 64 * 64;
    r = (int)(per < 64 ? 64 : std::min<int64_t>(per, 1 << 20));
  }
  r = (r + 15) / 16 * 16;
  if (r > 2048) r = 2048;
  if (r < 16) r = 16;
  return r;
}
// Keys per scoring workgroup (512, 2048 and 4096 measured slower at 128K).
static int decode_score_rows() { return 1024; }

struct DecodePlan {
  int64_t kk;
  int score_rows, n_score_chunks, n_sel_chunks, split_rows, nsplit;
  size_t off_logits, off_stats, off_pooled, off_hist, off_counts, off_selstate, off_cand, off_part_o,
      off_part_ml, off_prow, off_pos, total;
};

// dense: the split rows cover the whole cache (kk = N) and only the split
// partials are needed. paged: room for the physical rows of the call's sets
// (Hkv sets of kk rows per batch row; dense: one set of all N keys).
// kk_fixed > 0: the sets hold that many keys (a refined layer's kappa; s.N is
// then the pool size) and room for the selected pool positions is added.
static DecodePlan plan_decode(const Shape& s, bool anchor, bool dense = false, bool paged = false,
                              int64_t kk_fixed = 0) {
  DecodePlan p{};
  p.kk = kk_fixed > 0 ? kk_fixed : (dense ? s.N : decode_k(s.N, s.pct));
  p.score_rows = decode_score_rows();
  p.n_score_chunks = (int)((s.N + p.score_rows - 1) / p.score_rows);
  p.n_sel_chunks = (int)((s.N + kSelChunk - 1) / kSelChunk);
  p.split_rows = decode_split_rows((int64_t)s.B * s.Hkv, p.kk);
  p.nsplit = (int)((p.kk + p.split_rows - 1) / p.split_rows);
  const size_t units = (size_t)s.B * s.Hkv;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes, 256); return o; };
  if (anchor) {
    p.off_logits = take(units * s.N * s.G * sizeof(float));
    p.off_stats = take(units * p.n_score_chunks * s.G * 2 * sizeof(float));
    p.off_pooled = take(units * ((s.N + 3) / 4 * 4) * sizeof(float));
    p.off_hist = take(units * kHistWords * sizeof(uint32_t));
    p.off_counts = take(units * p.n_sel_chunks * 2 * sizeof(uint32_t));
    p.off_selstate = take(units * 4 * sizeof(uint32_t));
    p.off_cand = take(units * p.n_sel_chunks * kSelChunk * sizeof(uint32_t));
  }
  p.off_part_o = take((size_t)s.B * s.Hq * p.nsplit * s.D * sizeof(float));
  p.off_part_ml = take((size_t)s.B * s.Hq * p.nsplit * 2 * sizeof(float));
  if (paged) p.off_prow = take((size_t)s.B * (dense ? 1 : s.Hkv) * p.kk * sizeof(uint32_t));
  if (kk_fixed > 0) p.off_pos = take((size_t)s.B * s.Hkv * p.kk * sizeof(int32_t));
  p.total = off;
  return p;
}

// A checked kas_kv_cache_t (all zero: the dense cache of the descriptor).
struct CacheView {
  const int32_t* seq_lens = nullptr;
  const int32_t* block_table = nullptr;
  int shift = 0, max_pages = 0;
  int64_t num_pages = 0, page_stride = 0, page_hstride = 0, pool_rows = 0;
  bool paged() const { return block_table != nullptr; }
};

static kas_status_t check_cache(const kas_kv_cache_t* c, const Shape& s, CacheView& v) {
  v = CacheView{};
  if (!c) return KAS_OK;
  v.seq_lens = c->seq_lens;
  if (!c->block_table) return KAS_OK;
  if (s.dtype == KAS_DTYPE_F32) return fail(KAS_ERR_UNSUPPORTED, "paged caches hold bf16 or fp16");
  const int64_t P = c->page_size;
  if (P < 16 || P > (1 << 20) || (P & (P - 1)))
    return fail(KAS_ERR_INVALID_ARGUMENT, "page_size must be a power of two in [16, 2^20] (got %lld)", (long long)P);
  if (c->max_pages < (s.N + P - 1) / P)
    return fail(KAS_ERR_INVALID_ARGUMENT, "max_pages (%d) does not cover seq_len %lld", c->max_pages, (long long)s.N);
  if (c->num_pages < 1) return fail(KAS_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  const int64_t phs = c->page_head_stride ? c->page_head_stride : P * s.D;
  const int64_t ps = c->page_stride ? c->page_stride : s.Hkv * P * s.D;
  if (phs < P * s.D || ps < (s.Hkv - 1) * phs + P * s.D)
    return fail(KAS_ERR_INVALID_ARGUMENT, "page strides overlap the [P, D] rows of a head");
  const int64_t vec = 16 / (int64_t)s.esize;
  if (ps % vec || phs % vec) return fail(KAS_ERR_INVALID_ARGUMENT, "page strides must be multiples of 16 bytes");
  if (ps % s.D) return fail(KAS_ERR_INVALID_ARGUMENT, "page_stride must be a multiple of head_dim");
  const int64_t rows = c->num_pages * (ps / s.D);
  if (rows >= (int64_t(1) << 31) || c->num_pages >= (int64_t(1) << 31))
    return fail(KAS_ERR_UNSUPPORTED, "page pool of %lld rows: 2^31 or more", (long long)rows);
  v.block_table = c->block_table;
  int shift = 0;
  while ((int64_t(1) << shift) < P) ++shift;
  v.shift = shift;
  v.max_pages = c->max_pages;
  v.num_pages = c->num_pages;
  v.page_stride = ps;
  v.page_hstride = phs;
  v.pool_rows = rows;
  return KAS_OK;
}

static void fill_cache(DecodeArgs& a, const CacheView& v, const Shape& s) {
  a.seq_lens = v.seq_lens;
  a.pct = s.pct;
  a.block_table = v.block_table;
  a.page_shift = v.shift;
  a.max_pages = v.max_pages;
  a.num_pages = v.num_pages;
  a.page_stride = v.page_stride;
  a.page_hstride = v.page_hstride;
  a.pool_rows = v.pool_rows;
}

// The reuse shape with one anchor set per query head: the gather kernels run
// every query head as its own group of one (Hkv = Hq, G = 1) and address K and
// V through head / G.
static Shape per_query_head(const Shape& s) {
  Shape q = s;
  q.Hkv = s.Hq;
  q.G = 1;
  return q;
}

static void fill_decode_args(const Shape& s, const DecodePlan& p, bool anchor, char* ws, DecodeArgs& a) {
  memset(&a, 0, sizeof(a));
  a.kvdiv = 1;
  a.kv_bstride = s.kv_bs; a.kv_hstride = s.kv_hs;
  a.q_bstride = s.q_bs; a.q_hstride = s.q_hs;
  a.o_bstride = s.o_bs; a.o_hstride = s.o_hs;
  a.B = s.B; a.Hq = s.Hq; a.Hkv = s.Hkv; a.D = s.D; a.G = s.G; a.N = s.N;
  a.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
  a.kk = p.kk;
  a.pstride = (s.N + 3) / 4 * 4;
  a.score_rows = p.score_rows; a.n_score_chunks = p.n_score_chunks; a.n_sel_chunks = p.n_sel_chunks;
  a.split_rows = p.split_rows; a.nsplit = p.nsplit;
  a.pool_op = s.op; a.pool_all = s.scope;
  a.sel_units = (int64_t)s.B * (s.scope ? 1 : s.Hkv);
  if (anchor) {
    a.logits = (float*)(ws + p.off_logits);
    a.stats = (float*)(ws + p.off_stats);
    a.pooled = (float*)(ws + p.off_pooled);
    a.hist = (uint32_t*)(ws + p.off_hist);
    a.counts = (uint32_t*)(ws + p.off_counts);
    a.selstate = (uint32_t*)(ws + p.off_selstate);
    a.cand = (uint32_t*)(ws + p.off_cand);
  }
  a.part_o = (float*)(ws + p.off_part_o);
  a.part_ml = (float*)(ws + p.off_part_ml);
  a.prow = p.off_prow ? (uint32_t*)(ws + p.off_prow) : nullptr;
}

static kas_status_t check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(KAS_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  if (need && !ws) return fail(KAS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (need && ((uintptr_t)ws & 255u)) return fail(KAS_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return KAS_OK;
}

// The prefill kernels keep CSR offsets and index positions in 32 bits and
// address a KV head's rows through 32-bit byte offsets.
static kas_status_t check_prefill_limits(const Shape& s, int64_t total) {
  if (total > INT32_MAX)
    return fail(KAS_ERR_UNSUPPORTED, "prefill index set of %lld entries per KV head exceeds 2^31 - 1",
                (long long)total);
  if (s.N * 2 * s.D > INT32_MAX)
    return fail(KAS_ERR_UNSUPPORTED, "prefill KV head slice of %lld bytes reaches 2^31",
                (long long)(s.N * 2 * s.D));
  return KAS_OK;
}

// Prefill calls take a kas_kv_cache_t for prompts of different lengths and
// for paged pools. A paged call first copies its prompts' K and V rows, page
// by page, into contiguous [B, Hkv, N, D] copies placed after the call's own
// workspace, and the tile kernels read those: the tile kernels are bound by
// their matrix products, so one more pass over K and V costs little, and their
// DMA pipelines keep plain row offsets.
static size_t paged_copy_bytes(const Shape& s) {
  return align_up((size_t)s.B * s.Hkv * (size_t)s.N * s.D * s.esize, 256);
}

static size_t prefill_need(size_t base, const Shape& s, const CacheView& cv) {
  return cv.paged() ? align_up(base, 256) + 2 * paged_copy_bytes(s) : base;
}

// Copies a paged call's K and V (s: the call's own shape, with its KV heads)
// and points the tile kernels' arguments at the copies.
static hipError_t prefill_paged_kv(const CacheView& cv, const Shape& s, const void* k, const void* v, char* ws,
                                   size_t base, PrefillArgs& a, LaunchCtx& ctx) {
  PageCopyArgs c{};
  c.k = k; c.v = v;
  c.kc = ws + align_up(base, 256);
  c.vc = (char*)c.kc + paged_copy_bytes(s);
  c.seq_lens = cv.seq_lens; c.block_table = cv.block_table;
  c.page_stride = cv.page_stride; c.page_hstride = cv.page_hstride; c.num_pages = cv.num_pages;
  c.N = s.N; c.B = s.B; c.Hkv = s.Hkv; c.D = s.D; c.T = (int)(s.N / 32);
  c.shift = cv.shift; c.max_pages = cv.max_pages;
  a.k = c.kc; a.v = c.vc;
  a.kv_hstride = s.N * s.D;
  a.kv_bstride = (int64_t)s.Hkv * s.N * s.D;
  return launch_prefill_page_copy(c, ctx);
}

static void set_qo_strides(PrefillArgs& a, const Shape& s) {
  a.q_bstride = s.q_bs; a.q_hstride = s.q_hs; a.q_tstride = s.q_ts;
  a.o_bstride = s.o_bs; a.o_hstride = s.o_hs; a.o_tstride = s.o_ts;
}

static kas_status_t hip_fail(hipError_t e, const char* where) {
  return fail(KAS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ------------------------------------------------------------------ static scratch

// The buffer of kas_decode_reuse_noalloc. In host code `scratch` names a
// host-side stand-in, not device memory: only the address that
// hipGetSymbolAddress returns for the current device is passed on.
static __device__ __align__(256) char scratch[KAS_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

// This device's copy of the static buffer, looked up once per device.
static kas_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(KAS_ERR_UNSUPPORTED, "device %d: at most 64 devices", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || ((uintptr_t)ptr & 255u)) return fail(KAS_ERR_HIP, "static scratch buffer has no aligned address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KAS_OK;
}

}  // namespace kas

using namespace kas;

// ------------------------------------------------------------------ exported

extern "C" {

int64_t kas_topk_count(int64_t n, int32_t pct) { return kas::topk_count(n, pct); }

kas_status_t kas_prefill_index_offsets(const kas_desc_t* desc, int64_t* offsets, int64_t* total) {
  Shape s;
  kas_status_t st = check_desc(desc, true, s);
  if (st != KAS_OK) return st;
  if (!total) return fail(KAS_ERR_INVALID_ARGUMENT, "total is NULL");
  const int64_t T = s.N / s.tile;
  int64_t acc = 0;
  for (int64_t t = 0; t < T; ++t) {
    if (offsets) offsets[t] = acc;
    acc += kas::topk_count(t * s.tile, s.pct);
  }
  if (offsets) offsets[T] = acc;
  *total = acc;
  if (acc >= (int64_t(1) << 31)) return fail(KAS_ERR_UNSUPPORTED, "index set larger than 2^31 entries");
  return KAS_OK;
}

// An anchor call's workspace: its own plan, or with a dense output the larger
// of that and the dense plan (the dense output runs after the selection and
// reuses the workspace from its start).
static size_t decode_anchor_need(const Shape& s, bool paged) {
  size_t need = plan_decode(s, true, false, paged).total;
  if (s.dense_out) need = std::max(need, plan_decode(s, false, true, paged).total);
  return need;
}

// Dense decode attention over every key of each sequence: split-K gather
// over the keys (paged: their physical rows first) and the merge.
static hipError_t run_decode_dense(const Shape& s, const CacheView& cv, const void* q, const void* k, const void* v,
                                   void* o, char* ws, LaunchCtx& ctx, const char** where) {
  const DecodePlan p = plan_decode(s, false, true, cv.paged());
  DecodeArgs a;
  fill_decode_args(s, p, false, ws, a);
  fill_cache(a, cv, s);
  a.rows_are_keys = 1;       // a sequence's "set" is all its keys
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.idx = nullptr; a.Hkv_a = s.Hkv; a.head_map = nullptr;
  hipError_t e;
  if (cv.paged()) {
    a.page_src = nullptr;
    a.page_src_sets = 1;
    *where = "decode_page_rows";
    if ((e = launch_page_rows(a, 1, ctx)) != hipSuccess) return e;
    a.idx = (const int32_t*)a.prow; a.Hkv_a = 1;
  }
  *where = "decode_dense";
  return launch_decode_dense(a, s.dtype, ctx);
}

kas_status_t kas_workspace_size(const kas_desc_t* desc, int32_t op, size_t* bytes) {
  return kas_workspace_size_kv(desc, nullptr, op, bytes);
}

kas_status_t kas_workspace_size_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, int32_t op, size_t* bytes) {
  if (!bytes) return fail(KAS_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Shape s;
  const bool prefill = op == KAS_OP_PREFILL_ANCHOR || op == KAS_OP_PREFILL_REUSE || op == KAS_OP_PREFILL_DENSE;
  if (op < KAS_OP_DECODE_ANCHOR || op > KAS_OP_PREFILL_DENSE) return fail(KAS_ERR_INVALID_ARGUMENT, "unknown op %d", op);
  kas_status_t st = check_desc(desc, prefill, s);
  if (st != KAS_OK) return st;
  CacheView cv;
  if ((st = check_cache(cache, s, cv))) return st;
  if (op == KAS_OP_PREFILL_DENSE) {
    *bytes = prefill_need(0, s, cv);
  } else if (op == KAS_OP_DECODE_REUSE && s.qmap) {
    *bytes = plan_decode(per_query_head(s), false, false, cv.paged()).total;
  } else if (op == KAS_OP_DECODE_ANCHOR) {
    *bytes = decode_anchor_need(s, cv.paged());
  } else if (!prefill) {
    *bytes = plan_decode(s, false, op == KAS_OP_DECODE_DENSE, cv.paged()).total;
  } else {
    const Shape sr = (op == KAS_OP_PREFILL_REUSE && s.qmap) ? per_query_head(s) : s;
    *bytes = prefill_need(prefill_workspace_bytes(sr.B, sr.Hq, sr.Hkv, sr.D, sr.N, sr.pct, op == KAS_OP_PREFILL_ANCHOR),
                          s, cv);
  }
  return KAS_OK;
}

kas_status_t kas_decode_anchor(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                               int32_t* idx_out, void* o, void* ws, size_t ws_bytes, void* stream) {
  return kas_decode_anchor_kv(desc, nullptr, q, k, v, idx_out, o, ws, ws_bytes, stream);
}

kas_status_t kas_decode_anchor_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, int32_t* idx_out, void* o, void* ws,
                                  size_t ws_bytes, void* stream) {
  Shape s;
  kas_status_t st = check_desc(desc, false, s);
  if (st != KAS_OK) return st;
  CacheView cv;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if (!idx_out) return fail(KAS_ERR_INVALID_ARGUMENT, "idx_out is NULL");
  DecodePlan p = plan_decode(s, true, false, cv.paged());
  if ((st = check_ws(ws, ws_bytes, decode_anchor_need(s, cv.paged())))) return st;
  DecodeArgs a;
  fill_decode_args(s, p, true, (char*)ws, a);
  fill_cache(a, cv, s);
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.idx_out = idx_out;
  // the output reads the selected sets back: one per KV head, or one shared
  a.idx = idx_out; a.Hkv_a = s.scope ? 1 : s.Hkv; a.head_map = nullptr;
  LaunchCtx ctx{(hipStream_t)stream};
  hipError_t e;
  if ((e = launch_decode_score(a, s.dtype, ctx)) != hipSuccess) return hip_fail(e, "decode_score");
  if ((e = launch_decode_pool(a, ctx)) != hipSuccess) return hip_fail(e, "decode_pool");
  if ((e = launch_decode_select(a, ctx)) != hipSuccess) return hip_fail(e, "decode_select");
  if (s.dense_out) {
    const char* where = "decode_dense";
    if ((e = run_decode_dense(s, cv, q, k, v, o, (char*)ws, ctx, &where)) != hipSuccess) return hip_fail(e, where);
    return KAS_OK;
  }
  if (cv.paged()) {
    // physical rows of every KV head's set, then the output from them
    a.page_src = idx_out;
    a.page_src_sets = a.Hkv_a;
    if ((e = launch_page_rows(a, s.Hkv, ctx)) != hipSuccess) return hip_fail(e, "decode_page_rows");
    a.idx = (const int32_t*)a.prow; a.Hkv_a = s.Hkv;
  }
  if ((e = launch_decode_attn(a, s.dtype, true, ctx)) != hipSuccess) return hip_fail(e, "decode_attn");
  return KAS_OK;
}

kas_status_t kas_decode_reuse(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                              const int32_t* anchor_idx, int32_t anchor_kv_heads,
                              const int32_t* head_map, void* o, void* ws, size_t ws_bytes,
                              void* stream) {
  return kas_decode_reuse_kv(desc, nullptr, q, k, v, anchor_idx, anchor_kv_heads, head_map, o, ws, ws_bytes,
                             stream);
}

kas_status_t kas_decode_reuse_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                 const void* k, const void* v, const int32_t* anchor_idx,
                                 int32_t anchor_kv_heads, const int32_t* head_map, void* o, void* ws,
                                 size_t ws_bytes, void* stream) {
  Shape s;
  kas_status_t st = check_desc(desc, false, s);
  if (st != KAS_OK) return st;
  CacheView cv;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if (!anchor_idx) return fail(KAS_ERR_INVALID_ARGUMENT, "anchor_idx is NULL");
  if (anchor_kv_heads < 1) return fail(KAS_ERR_INVALID_ARGUMENT, "anchor_kv_heads must be >= 1");
  if (!head_map && anchor_kv_heads != s.Hkv && anchor_kv_heads != 1)
    return fail(KAS_ERR_INVALID_ARGUMENT,
                "without a head map, anchor_kv_heads must be n_kv_heads (identity) or 1 (shared set)");
  if (s.qmap && !head_map) return fail(KAS_ERR_INVALID_ARGUMENT, "query_head_map needs a head_map of n_q_heads entries");
  const Shape sr = s.qmap ? per_query_head(s) : s;
  DecodePlan p = plan_decode(sr, false, false, cv.paged());
  if ((st = check_ws(ws, ws_bytes, p.total))) return st;
  DecodeArgs a;
  fill_decode_args(sr, p, false, (char*)ws, a);
  fill_cache(a, cv, s);
  a.kvdiv = s.qmap ? s.G : 1;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.idx = anchor_idx; a.Hkv_a = anchor_kv_heads; a.head_map = head_map;
  LaunchCtx ctx{(hipStream_t)stream};
  hipError_t e;
  if (cv.paged()) {
    // this layer's sets (head map applied) as physical rows
    a.page_src = anchor_idx;
    a.page_src_sets = anchor_kv_heads;
    if ((e = launch_page_rows(a, sr.Hkv, ctx)) != hipSuccess) return hip_fail(e, "decode_page_rows");
    a.idx = (const int32_t*)a.prow; a.Hkv_a = sr.Hkv; a.head_map = nullptr;
  }
  if ((e = launch_decode_attn(a, s.dtype, false, ctx)) != hipSuccess) return hip_fail(e, "decode_attn");
  return KAS_OK;
}

kas_status_t kas_decode_reuse_noalloc(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                                      const int32_t* anchor_idx, int32_t anchor_kv_heads, const int32_t* head_map,
                                      void* o, void* stream) {
  size_t need = 0;
  kas_status_t st = kas_workspace_size(desc, KAS_OP_DECODE_REUSE, &need);
  if (st != KAS_OK) return st;
  // the argument checks of kas_decode_reuse come first, before any device query
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if (!anchor_idx) return fail(KAS_ERR_INVALID_ARGUMENT, "anchor_idx is NULL");
  if (anchor_kv_heads < 1) return fail(KAS_ERR_INVALID_ARGUMENT, "anchor_kv_heads must be >= 1");
  if (need > KAS_NOALLOC_SCRATCH_BYTES)
    return fail(KAS_ERR_UNSUPPORTED, "decode reuse needs %zu bytes of scratch; the static buffer holds %u",
                need, (unsigned)KAS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != KAS_OK) return st;
  return kas_decode_reuse_kv(desc, nullptr, q, k, v, anchor_idx, anchor_kv_heads, head_map, o, ws,
                             KAS_NOALLOC_SCRATCH_BYTES, stream);
}

kas_status_t kas_prefill_anchor(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                                int32_t* idx_out, void* o, void* ws, size_t ws_bytes, void* stream) {
  return kas_prefill_anchor_kv(desc, nullptr, q, k, v, idx_out, o, ws, ws_bytes, stream);
}

kas_status_t kas_prefill_anchor_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                   const void* k, const void* v, int32_t* idx_out, void* o, void* ws,
                                   size_t ws_bytes, void* stream) {
  Shape s;
  kas_status_t st = check_desc(desc, true, s);
  if (st != KAS_OK) return st;
  CacheView cv;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if (!idx_out) return fail(KAS_ERR_INVALID_ARGUMENT, "idx_out is NULL");
  int64_t total = 0;
  if ((st = kas_prefill_index_offsets(desc, nullptr, &total))) return st;
  if ((st = check_prefill_limits(s, total))) return st;
  const size_t base = prefill_workspace_bytes(s.B, s.Hq, s.Hkv, s.D, s.N, s.pct, true);
  if ((st = check_ws(ws, ws_bytes, prefill_need(base, s, cv)))) return st;
  PrefillArgs a;
  fill_prefill_args(a, s.B, s.Hq, s.Hkv, s.D, s.N, s.pct, s.scale, s.kv_bs, s.kv_hs, (char*)ws, true);
  set_qo_strides(a, s);
  a.dtype = s.dtype;
  a.q = q; a.k = k; a.v = v; a.o = o; a.idx_out = idx_out;
  a.pool_op = s.op; a.pool_all = s.scope; a.Hsel = s.scope ? 1 : s.Hkv;
  a.idx = idx_out; a.Hkv_a = a.Hsel; a.head_map = nullptr; a.total = total;
  a.seq_lens = cv.seq_lens;
  a.dense_out = s.dense_out;
  LaunchCtx ctx{(hipStream_t)stream};
  hipError_t e;
  if (cv.paged() && (e = prefill_paged_kv(cv, s, k, v, (char*)ws, base, a, ctx)) != hipSuccess)
    return hip_fail(e, "prefill_page_copy");
  e = launch_prefill_anchor(a, ctx);
  if (e != hipSuccess) return hip_fail(e, "prefill_anchor");
  return KAS_OK;
}

kas_status_t kas_prefill_reuse(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                               const int32_t* anchor_idx, int32_t anchor_kv_heads,
                               const int32_t* head_map, void* o, void* ws, size_t ws_bytes,
                               void* stream) {
  return kas_prefill_reuse_kv(desc, nullptr, q, k, v, anchor_idx, anchor_kv_heads, head_map, o, ws, ws_bytes,
                              stream);
}

kas_status_t kas_prefill_reuse_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, const int32_t* anchor_idx,
                                  int32_t anchor_kv_heads, const int32_t* head_map, void* o, void* ws,
                                  size_t ws_bytes, void* stream) {
  Shape s;
  kas_status_t st = check_desc(desc, true, s);
  if (st != KAS_OK) return st;
  CacheView cv;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if (!anchor_idx) return fail(KAS_ERR_INVALID_ARGUMENT, "anchor_idx is NULL");
  if (anchor_kv_heads < 1) return fail(KAS_ERR_INVALID_ARGUMENT, "anchor_kv_heads must be >= 1");
  if (!head_map && anchor_kv_heads != s.Hkv && anchor_kv_heads != 1)
    return fail(KAS_ERR_INVALID_ARGUMENT,
                "without a head map, anchor_kv_heads must be n_kv_heads (identity) or 1 (shared set)");
  int64_t total = 0;
  if ((st = kas_prefill_index_offsets(desc, nullptr, &total))) return st;
  if ((st = check_prefill_limits(s, total))) return st;
  if (s.qmap && !head_map) return fail(KAS_ERR_INVALID_ARGUMENT, "query_head_map needs a head_map of n_q_heads entries");
  const Shape sr = s.qmap ? per_query_head(s) : s;
  const size_t base = prefill_workspace_bytes(sr.B, sr.Hq, sr.Hkv, sr.D, sr.N, sr.pct, false);
  if ((st = check_ws(ws, ws_bytes, prefill_need(base, s, cv)))) return st;
  PrefillArgs a;
  fill_prefill_args(a, sr.B, sr.Hq, sr.Hkv, sr.D, sr.N, sr.pct, sr.scale, sr.kv_bs, sr.kv_hs, (char*)ws, false);
  set_qo_strides(a, sr);
  a.dtype = s.dtype;
  a.kvdiv = s.qmap ? s.G : 1;
  a.seq_lens = cv.seq_lens;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.idx = anchor_idx; a.Hkv_a = anchor_kv_heads; a.head_map = head_map; a.total = total;
  LaunchCtx ctx{(hipStream_t)stream};
  hipError_t e;
  if (cv.paged() && (e = prefill_paged_kv(cv, s, k, v, (char*)ws, base, a, ctx)) != hipSuccess)
    return hip_fail(e, "prefill_page_copy");
  e = launch_prefill_reuse(a, ctx);
  if (e != hipSuccess) return hip_fail(e, "prefill_reuse");
  return KAS_OK;
}

kas_status_t kas_decode_dense(const kas_desc_t* desc, const void* q, const void* k, const void* v, void* o,
                              void* ws, size_t ws_bytes, void* stream) {
  return kas_decode_dense_kv(desc, nullptr, q, k, v, o, ws, ws_bytes, stream);
}

kas_status_t kas_decode_dense_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                 const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                                 void* stream) {
  Shape s;
  kas_status_t st = check_desc(desc, false, s);
  if (st != KAS_OK) return st;
  CacheView cv;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if ((st = check_ws(ws, ws_bytes, plan_decode(s, false, true, cv.paged()).total))) return st;
  LaunchCtx ctx{(hipStream_t)stream};
  const char* where = "decode_dense";
  hipError_t e = run_decode_dense(s, cv, q, k, v, o, (char*)ws, ctx, &where);
  if (e != hipSuccess) return hip_fail(e, where);
  return KAS_OK;
}

kas_status_t kas_prefill_dense(const kas_desc_t* desc, const void* q, const void* k, const void* v, void* o,
                               void* ws, size_t ws_bytes, void* stream) {
  return kas_prefill_dense_kv(desc, nullptr, q, k, v, o, ws, ws_bytes, stream);
}

kas_status_t kas_prefill_dense_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                                  void* stream) {
  Shape s;
  kas_status_t st = check_desc(desc, true, s);
  if (st != KAS_OK) return st;
  CacheView cv;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if ((st = check_prefill_limits(s, 0))) return st;
  if ((st = check_ws(ws, ws_bytes, prefill_need(0, s, cv)))) return st;   // 0 bytes unless paged
  PrefillArgs a;
  fill_prefill_args(a, s.B, s.Hq, s.Hkv, s.D, s.N, s.pct, s.scale, s.kv_bs, s.kv_hs, nullptr, false);
  set_qo_strides(a, s);
  a.dtype = s.dtype;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.offsets = nullptr; a.idx = nullptr; a.Hkv_a = s.Hkv; a.head_map = nullptr; a.total = 0;
  a.seq_lens = cv.seq_lens;
  LaunchCtx ctx{(hipStream_t)stream};
  hipError_t e;
  if (cv.paged() && (e = prefill_paged_kv(cv, s, k, v, (char*)ws, 0, a, ctx)) != hipSuccess)
    return hip_fail(e, "prefill_page_copy");
  e = launch_prefill_dense(a, ctx);
  if (e != hipSuccess) return hip_fail(e, "prefill_dense");
  return KAS_OK;
}

// Refined layer of proposal-refined reuse: the pool-sized plan (scores,
// pooled values and selection over the pool; gather splits over kappa). With
// one set per query head the plan is that of the per-query-head shape. A
// paged cache adds the pool's physical rows (B * sets * pool_size) after it;
// every plan ends with room for the per-sequence pool sizes and kappas.
static kas_status_t refine_plan(const Shape& s, int64_t pool_size, Shape& sp, DecodePlan& p, bool paged,
                                size_t* off_pool_rows = nullptr, size_t* off_lens = nullptr) {
  const int64_t kappa = decode_k(s.N, s.pct);
  if (pool_size < kappa || pool_size > s.N)
    return fail(KAS_ERR_INVALID_ARGUMENT, "pool_size %lld must lie in [kappa = %lld, seq_len = %lld]",
                (long long)pool_size, (long long)kappa, (long long)s.N);
  if (s.scope || s.op)
    return fail(KAS_ERR_UNSUPPORTED, "refined layers pool by sum within each set (pool_scope and pool_op 0)");
  sp = s.qmap ? per_query_head(s) : s;
  sp.N = pool_size;
  p = plan_decode(sp, true, false, paged, kappa);
  size_t off = p.total;
  if (paged) {
    if (off_pool_rows) *off_pool_rows = off;
    off = align_up(off + (size_t)s.B * sp.Hkv * pool_size * sizeof(uint32_t), 256);
  }
  if (off_lens) *off_lens = off;
  p.total = align_up(off + (size_t)2 * s.B * sizeof(int32_t), 256);
  return KAS_OK;
}

kas_status_t kas_workspace_size_refine(const kas_desc_t* desc, int64_t pool_size, size_t* bytes) {
  return kas_workspace_size_refine_kv(desc, nullptr, pool_size, bytes);
}

kas_status_t kas_workspace_size_refine_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, int64_t pool_size,
                                          size_t* bytes) {
  if (!bytes) return fail(KAS_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Shape s, sp;
  DecodePlan p;
  CacheView cv;
  kas_status_t st = check_desc(desc, false, s);
  if (st != KAS_OK) return st;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = refine_plan(s, pool_size, sp, p, cv.paged()))) return st;
  *bytes = p.total;
  return KAS_OK;
}

kas_status_t kas_decode_refine(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                               const int32_t* pool_idx, int32_t pool_kv_heads, int64_t pool_size,
                               const int32_t* head_map, int32_t* idx_out, void* o, void* ws,
                               size_t ws_bytes, void* stream) {
  return kas_decode_refine_kv(desc, nullptr, q, k, v, pool_idx, pool_kv_heads, pool_size, nullptr, head_map,
                              idx_out, o, ws, ws_bytes, stream);
}

kas_status_t kas_decode_refine_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, const int32_t* pool_idx, int32_t pool_kv_heads,
                                  int64_t pool_size, const int32_t* pool_lens, const int32_t* head_map,
                                  int32_t* idx_out, void* o, void* ws, size_t ws_bytes, void* stream) {
  Shape s, sp;
  DecodePlan p;
  CacheView cv;
  size_t off_pool_rows = 0, off_lens = 0;
  kas_status_t st = check_desc(desc, false, s);
  if (st != KAS_OK) return st;
  if ((st = check_cache(cache, s, cv))) return st;
  if ((st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) || (st = check_ptr(v, "v")) ||
      (st = check_ptr(o, "o")))
    return st;
  if (!pool_idx) return fail(KAS_ERR_INVALID_ARGUMENT, "pool_idx is NULL");
  if (!idx_out) return fail(KAS_ERR_INVALID_ARGUMENT, "idx_out is NULL");
  if (pool_kv_heads < 1) return fail(KAS_ERR_INVALID_ARGUMENT, "pool_kv_heads must be >= 1");
  if (s.qmap && !head_map) return fail(KAS_ERR_INVALID_ARGUMENT, "query_head_map needs a head_map of n_q_heads entries");
  if (!head_map && pool_kv_heads != s.Hkv && pool_kv_heads != 1)
    return fail(KAS_ERR_INVALID_ARGUMENT,
                "without a head map, pool_kv_heads must be n_kv_heads (identity) or 1 (shared pool)");
  if ((st = refine_plan(s, pool_size, sp, p, cv.paged(), &off_pool_rows, &off_lens))) return st;
  if ((st = check_ws(ws, ws_bytes, p.total))) return st;
  const int sets = sp.Hkv;     // Hkv, or Hq with one set per query head
  DecodeArgs a;
  fill_decode_args(sp, p, true, (char*)ws, a);
  fill_cache(a, cv, s);
  a.kvdiv = s.qmap ? s.G : 1;
  a.q = q; a.k = k; a.v = v; a.o = o;
  LaunchCtx ctx{(hipStream_t)stream};
  hipError_t e;
  // sequences of different lengths or pools: sequence b's pool size and kappa
  const bool varlen = cv.seq_lens || pool_lens;
  int32_t* lens_pool = (int32_t*)((char*)ws + off_lens);
  int32_t* lens_kappa = lens_pool + s.B;
  if (varlen && (e = launch_refine_lens(cv.seq_lens, pool_lens, s.B, s.N, pool_size, s.pct, lens_pool, lens_kappa,
                                        ctx)) != hipSuccess)
    return hip_fail(e, "decode_refine_lens");
  const int32_t* set_lens = varlen ? lens_kappa : nullptr;
  if (cv.paged()) {
    // the pools' keys (head map applied) as physical rows, scored from there
    DecodeArgs t = a;
    t.N = s.N; t.kk = pool_size;
    t.seq_lens = cv.seq_lens; t.set_lens = varlen ? lens_pool : nullptr;
    t.prow = (uint32_t*)((char*)ws + off_pool_rows);
    t.page_src = pool_idx; t.page_src_sets = pool_kv_heads; t.head_map = head_map;
    if ((e = launch_page_rows(t, sets, ctx)) != hipSuccess) return hip_fail(e, "decode_page_rows");
    a.idx = (const int32_t*)t.prow; a.Hkv_a = sets; a.head_map = nullptr; a.n_keys = cv.pool_rows;
  } else {
    a.idx = pool_idx; a.Hkv_a = pool_kv_heads; a.head_map = head_map; a.n_keys = s.N;
  }
  // scoring, pooling and selection over the pool's keys: positions in the
  // pool (sequence b: its first pool_b positions, kappa_b kept)
  a.seq_lens = varlen ? lens_pool : nullptr;
  a.set_lens = set_lens;
  a.idx_out = (int32_t*)((char*)ws + p.off_pos);
  if ((e = launch_decode_score_pool_rows(a, s.dtype, ctx)) != hipSuccess) return hip_fail(e, "decode_score");
  if ((e = launch_decode_pool(a, ctx)) != hipSuccess) return hip_fail(e, "decode_pool");
  if ((e = launch_decode_select(a, ctx)) != hipSuccess) return hip_fail(e, "decode_select");
  // positions -> keys, then attention over the refined keys of the cache
  a.pos = a.idx_out;
  a.idx_out = idx_out;
  a.idx = pool_idx; a.Hkv_a = pool_kv_heads; a.head_map = head_map;
  if ((e = launch_pool_positions_to_keys(a, ctx)) != hipSuccess) return hip_fail(e, "decode_refine_map");
  DecodeArgs ga = a;
  ga.N = s.N;
  ga.seq_lens = cv.seq_lens; ga.set_lens = set_lens;
  ga.idx = idx_out; ga.Hkv_a = sets; ga.head_map = nullptr;
  if (cv.paged()) {
    ga.page_src = idx_out; ga.page_src_sets = sets;
    if ((e = launch_page_rows(ga, sets, ctx)) != hipSuccess) return hip_fail(e, "decode_page_rows");
    ga.idx = (const int32_t*)ga.prow;
  }
  if ((e = launch_decode_attn(ga, s.dtype, false, ctx)) != hipSuccess) return hip_fail(e, "decode_attn");
  return KAS_OK;
}

const char* kas_status_string(int32_t status) {
  switch (status) {
    case KAS_OK: return "ok";
    case KAS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KAS_ERR_UNSUPPORTED: return "unsupported";
    case KAS_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KAS_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* kas_last_error(void) { return kas::t_last_error.c_str(); }

kas_status_t kas_set_option(int32_t option, int64_t value) {
  if (option < 0 || option >= KAS_OPT_COUNT_) return fail(KAS_ERR_INVALID_ARGUMENT, "unknown option %d", option);
  if (value != -1) {
    bool ok = true;
    switch (option) {
      case KAS_OPT_DECODE_SPLIT_ROWS: ok = value >= 16 && value <= 2048; break;
      case KAS_OPT_DECODE_SELECT_ONE_PASS: ok = value == 0 || value == 1; break;
      case KAS_OPT_PREFILL_POOL_MB: ok = value >= 1 && value <= (int64_t(1) << 30); break;
      case KAS_OPT_PREFILL_SELECT_CAP: ok = value >= 0 && value <= 8192; break;
    }
    if (!ok) return fail(KAS_ERR_INVALID_ARGUMENT, "value %lld out of range for option %d", (long long)value, option);
  }
  kas::g_options[option].store(value, std::memory_order_relaxed);
  return KAS_OK;
}

kas_status_t kas_get_option(int32_t option, int64_t* value) {
  if (option < 0 || option >= KAS_OPT_COUNT_) return fail(KAS_ERR_INVALID_ARGUMENT, "unknown option %d", option);
  if (!value) return fail(KAS_ERR_INVALID_ARGUMENT, "value is NULL");
  *value = kas::g_options[option].load(std::memory_order_relaxed);
  return KAS_OK;
}

kas_status_t kas_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = enable != 0;
  return KAS_OK;
}

kas_status_t kas_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending_locked();
  for (int i = 0; i < K_COUNT_; ++i) { g_total_ms[i] = 0.0; g_launches[i] = 0; }
  return KAS_OK;
}

kas_status_t kas_profile_query(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(KAS_ERR_INVALID_ARGUMENT, "NULL argument");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  drain_pending_locked();
  for (int i = 0; i < K_COUNT_; ++i)
    if (!strcmp(kernel, kKernelNames[i])) {
      *total_ms = g_total_ms[i];
      *launches = g_launches[i];
      return KAS_OK;
    }
  return fail(KAS_ERR_INVALID_ARGUMENT, "unknown kernel name '%s'", kernel);
}

kas_status_t kas_profile_names(char* buf, size_t buf_len) {
  if (!buf || !buf_len) return fail(KAS_ERR_INVALID_ARGUMENT, "NULL buffer");
  std::string all;
  for (int i = 0; i < K_COUNT_; ++i) {
    if (i) all += ",";
    all += kKernelNames[i];
  }
  if (all.size() + 1 > buf_len) return fail(KAS_ERR_INVALID_ARGUMENT, "buffer too small");
  memcpy(buf, all.c_str(), all.size() + 1);
  return KAS_OK;
}

}  // extern "C"
