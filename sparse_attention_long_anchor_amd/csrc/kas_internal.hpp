// Internal launch interface between the C-ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "../../include/kascade.h"

namespace kas {

// Names under which kernel timings are reported (kas_profile_query).
enum KernelId {
  K_DEC_SCORE = 0,
  K_DEC_POOL,
  K_SEL_CAND,
  K_SEL_RESOLVE,
  K_SEL_COMPACT,
  K_SEL_FUSED,
  K_DEC_ATTN,
  K_DEC_ATTN_ANCHOR,
  K_DEC_COMBINE,
  K_PRE_STATS,
  K_PRE_POOL,
  K_PRE_SELECT,
  K_PRE_ATTN,
  K_DEC_DENSE,
  K_PRE_DENSE,
  K_PRE_POOL_HEADS,
  K_DEC_PAGE_ROWS,
  K_DEC_REFINE_MAP,
  K_DEC_REFINE_LENS,
  K_PRE_PAGE_COPY,
  K_COUNT_
};
const char* kernel_name(int id);

// Current value of a tuning option (kas_option_t), -1 when it is at its default.
int64_t option_value(int id);

// Wraps every launch: optional timing + launch error check. begin() takes a
// pair of events when profiling is on; launch() then passes them to the
// dispatch itself (hipExtLaunchKernel stamps the kernel's own start and end,
// adding no packets to the stream); end() files the pair for readout.
// Each begin/end bracket holds exactly one launch.
struct LaunchCtx {
  hipStream_t stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  void begin(int kid);
  hipError_t end(int kid);
  template <typename F, typename A>
  void launch(F kernel, dim3 grid, dim3 block, const A& arg) {
    if (e0) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, e0, e1, 0u, arg);
    else hipLaunchKernelGGL(kernel, grid, block, 0, stream, arg);
  }
};

// Radix-select digit layout over the fp32 bit pattern of a non-negative score:
// digit 1 = bits [31:21], digit 2 = bits [20:10], digit 3 = bits [9:0].
constexpr int kBins1 = 2048, kBins2 = 2048, kBins3 = 1024;
constexpr int kHistWords = kBins1 + kBins2 + kBins3;
constexpr int kSelChunk = 4096;         // scores per selection workgroup
constexpr int kMaxSelChunks = 4096;     // chunks the chunked selection resolves in LDS
constexpr int kMaxPoolHeads = 256;      // query heads one all-heads pooled set may cover
constexpr int kScoreMaxRows = 4096;     // keys per scoring workgroup (at most)

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t kv_bstride, kv_hstride;   // elements
  int64_t q_bstride, q_hstride;     // elements between batch rows / query heads of q
  int64_t o_bstride, o_hstride;     // the same for o
  int B, Hq, Hkv, D, G;
  int64_t N;
  float scale_log2;                 // softmax scale * log2(e)
  // index sets
  const int32_t* idx;               // [B, Hkv_a, kk]; unused by the dense kernels
  int64_t kk;
  int Hkv_a;
  const int32_t* head_map;          // [Hkv] or null
  int32_t* idx_out;                 // anchor: [B, Hkv, kk]
  // workspace regions
  float* logits;                    // [B, Hkv, N, G] base-2 logits
  float* stats;                     // [B, Hkv, n_score_chunks, G, 2]
  int n_score_chunks, score_rows;
  float* pooled;                    // [B, Hkv, pstride]
  int64_t pstride;                  // N rounded up to 4 (16-byte aligned rows)
  uint32_t* hist;                   // [B, Hkv, kHistWords]
  uint32_t* counts;                 // [B, Hkv, n_sel_chunks, 2]
  uint32_t* selstate;               // [B, Hkv, 4]: tau, r
  uint32_t* cand;                   // [B, Hkv, n_sel_chunks, kSelChunk]: candidate score bits
  int n_sel_chunks;
  float* part_o;                    // [B, Hq, nsplit, D]
  float* part_ml;                   // [B, Hq, nsplit, 2]
  int nsplit, split_rows;
  // selection variants: pooled score = sum (0) or max (1) of the heads'
  // probabilities; pool_all: one set per batch row over all heads
  int pool_op, pool_all;
  int64_t sel_units;                // index sets selected: B * Hkv, or B with pool_all
  // reuse with one anchor set per query head: Hkv and G describe query heads
  // (Hkv = Hq, G = 1) and KV head = head / kvdiv; 1 otherwise
  int kvdiv;
  // sequences of different lengths and paged caches
  const int32_t* seq_lens;          // [B] keys of sequence b (<= N), or null: all N
  int pct;                          // a sequence's set holds decode_k(seq_lens[b], pct) keys
  int rows_are_keys;                // gathers over whole sequences (dense): seq_lens[b] rows
  const int32_t* block_table;       // [B, max_pages] page of keys [P i, P i + P), or null
  int page_shift, max_pages;        // P = 1 << page_shift
  int64_t page_stride, page_hstride;  // elements between pages / between KV heads in a page
  int64_t pool_rows;                // paged: rows addressable from k + g * page_hstride
  int64_t num_pages;                // paged: pages in the pools (page ids are clamped to it)
  uint32_t* prow;                   // paged: physical rows of the sets this call gathers
  const int32_t* page_src;          // page-row translation: source sets, or null (keys 0..)
  int page_src_sets;                // sets per batch row in page_src
  // refined layer: scoring over a pool of keys (rows of a.idx through the
  // head map) instead of the cache; n_keys = rows of the cache
  int64_t n_keys;
  const int32_t* pos;               // selected positions in the pool [B, Hkv, kk]
  // refined layers over sequences of different lengths or pools: keys in
  // sequence b's sets (its kappa), or null: kk, or decode_k(seq_lens[b], pct)
  const int32_t* set_lens;
};

// Decode k of n keys: round-half-up(pct * n / 100) clamped to [1, n].
__host__ __device__ inline int64_t decode_k_of(int64_t n, int pct) {
  if (n <= 0 || pct <= 0) return n > 0 ? 1 : 0;
  int64_t k = ((int64_t)pct * n + 50) / 100;
  k = k > n ? n : k;
  return k < 1 ? 1 : k;
}

hipError_t launch_decode_score(const DecodeArgs& a, int dtype, LaunchCtx& ctx);
// Refined layer over sequences of different lengths or pools: for each b,
// pool_out[b] = pool_lens[b] (or pool_size) clamped to [1, min(pool_size,
// L_b)] and kappa_out[b] = min(decode_k(L_b, pct), pool_out[b]), with L_b =
// seq_lens[b] (or N) clamped to [1, N].
hipError_t launch_refine_lens(const int32_t* seq_lens, const int32_t* pool_lens, int B, int64_t N,
                              int64_t pool_size, int pct, int32_t* pool_out, int32_t* kappa_out, LaunchCtx& ctx);
hipError_t launch_decode_pool(const DecodeArgs& a, LaunchCtx& ctx);
hipError_t launch_decode_select(const DecodeArgs& a, LaunchCtx& ctx);
hipError_t launch_decode_attn(const DecodeArgs& a, int dtype, bool from_logits, LaunchCtx& ctx);
// Dense decode attention over all N keys: the split kernels with row i of a
// split standing for key split_rows * split + i (idx unused, kk = N).
hipError_t launch_decode_dense(const DecodeArgs& a, int dtype, LaunchCtx& ctx);
// Paged caches: physical rows of this call's sets into a.prow ([B, nsets,
// a.kk]); set s reads source set head_map[s] (or s, clamped) of a.page_src,
// or, with a.page_src null, the keys 0 .. seq_len - 1 themselves.
hipError_t launch_page_rows(const DecodeArgs& a, int nsets, LaunchCtx& ctx);
// Refined layer: Q.K^T and statistics over the pool rows (a.N = pool size);
// then the selected pool positions (a.pos) mapped to keys into a.idx_out.
hipError_t launch_decode_score_pool_rows(const DecodeArgs& a, int dtype, LaunchCtx& ctx);
hipError_t launch_pool_positions_to_keys(const DecodeArgs& a, LaunchCtx& ctx);

}  // namespace kas
