// Internal interface of the prefill kernels (tiles of 32 query rows).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kas_internal.hpp"

namespace kas {

constexpr int kTile = 32;

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int64_t kv_bstride, kv_hstride;   // elements
  int64_t q_bstride, q_hstride, q_tstride;   // elements between batch rows / query heads / tokens of q
  int64_t o_bstride, o_hstride, o_tstride;   // the same for o
  int B, Hq, Hkv, D, G, T, pct;
  int64_t N;
  float scale_log2;
  // index sets (CSR over tiles, per (b, KV head))
  const int32_t* idx;               // reuse: anchor sets [B, Hkv_a, total]
  int Hkv_a;
  const int32_t* head_map;
  int32_t* idx_out;                 // anchor: [B, Hkv, total]
  int64_t total;
  // workspace
  int32_t* offsets;                 // [T + 1]
  float* lse;                       // [B, Hq, N] base-2 log-sum-exp of each causal row
  float* pooled;                    // pooled rows of the current tile range
  size_t pooled_floats;             // capacity of `pooled`
  int t_begin, t_end;               // tile range of the current pool/select launch
  // per (b, KV head, tile): the first-digit bin of the k-th largest pooled
  // score, the count above it and the bin's size (int4), found by the pooling
  // pass; null when the rows change after pooling (pool_all), then the select
  // histograms the rows itself
  int32_t* sel_pre;
  int sel_cap;                      // select: largest first-digit bin resolved in LDS
  // selection variants: pooled score = sum (0) or max (1) over the tile's rows
  // and the heads; pool_all: one set per tile over all heads, Hsel sets per
  // (b, tile) in idx_out (Hkv, or 1 with pool_all)
  int pool_op, pool_all, Hsel;
  int dtype;                        // element type of q, k, v, o: 1 bf16, 2 fp16
  int kvdiv;                        // reuse per query head: Hkv = Hq, G = 1, KV head = head / kvdiv
  const int32_t* seq_lens;          // [B] prompt length of sequence b (tiles past it are skipped), or null
  int dense_out;                    // anchor: the output is dense causal attention (sets as usual)
};

size_t prefill_workspace_bytes(int B, int Hq, int Hkv, int D, int64_t N, int pct, bool anchor);
void fill_prefill_args(PrefillArgs& a, int B, int Hq, int Hkv, int D, int64_t N, int pct, float scale,
                       int64_t kv_bs, int64_t kv_hs, char* ws, bool anchor);
hipError_t launch_prefill_anchor(PrefillArgs& a, LaunchCtx& ctx);
hipError_t launch_prefill_reuse(PrefillArgs& a, LaunchCtx& ctx);
// Dense causal attention: tile t attends to keys [0, 32 t] block by block
// (idx, offsets and head_map unused).
hipError_t launch_prefill_dense(PrefillArgs& a, LaunchCtx& ctx);

// Prefill over a paged cache: the K and V rows of pools [pages, Hkv, P, D],
// read through a block table, into contiguous [B, Hkv, N, D] copies that the
// tile kernels above then read like any contiguous cache.
struct PageCopyArgs {
  const void* k;
  const void* v;                    // page pools
  void* kc;
  void* vc;                         // contiguous copies [B, Hkv, N, D]
  const int32_t* seq_lens;          // [B] or null: tiles past a prompt are not copied
  const int32_t* block_table;       // [B, max_pages] page ids (clamped to [0, num_pages))
  int64_t page_stride, page_hstride, num_pages;   // elements per page and per head in a page; pages
  int64_t N;
  int B, Hkv, D, T, shift, max_pages;             // shift = log2 of the page size
};
hipError_t launch_prefill_page_copy(const PageCopyArgs& c, LaunchCtx& ctx);

}  // namespace kas
