/*
 * kascade.h -- C ABI of the MI355X (gfx950) Kascade sparse-attention library.
 *
 * The method (Kascade README, "Abstract"): anchor layers compute exact Top-k
 * key indices from post-softmax attention scores; intermediate reuse layers
 * attend only over those indices; selection and reuse are head-aware; prefill
 * works on tiles of queries (README notes: tile size 32). One call of this
 * library is one attention layer of one kind (anchor or reuse) in one phase
 * (decode or prefill), the granularity of the README's kernel benchmarks
 * ("Kernel Benchmarks": --kernel recompute|reuse, decode and prefill).
 *
 * Conventions for every call
 *   - Pointers named q, k, v, o, idx, head_map, ws are DEVICE pointers; the
 *     caller allocates and owns them (including the workspace, sized by
 *     kas_workspace_size). The library never allocates device memory.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream) and
 *     is asynchronous; no call synchronises the stream.
 *   - All shape/argument checks run on the host before anything is enqueued;
 *     on failure nothing is enqueued and the status says why
 *     (kas_last_error() gives text, per calling thread).
 *   - Calls are thread-safe and keep no state between calls, except the
 *     optional kernel-timing registry (kas_profile_*) and the tuning options
 *     (kas_set_option).
 *   - Layouts are row-major with head_dim contiguous:
 *       decode : q, o [B, Hq, D];        k, v [B, Hkv, N, D]
 *       prefill: q, o [B, Hq, N, D];     k, v [B, Hkv, N, D]
 *     with the batch and head strides of q, o, k, v and the token strides of
 *     q and o given in kas_desc_t; the k and v rows of one head are adjacent.
 *     Query head h uses KV head h / (Hq / Hkv).
 *   - Index sets are int32 key positions in ascending order.
 *       decode : [B, Hs, kd]      kd = max(1, kas_topk_count(N, pct))
 *       prefill: [B, Hs, total]   CSR over query tiles; tile t's set is
 *                [offsets[t], offsets[t+1]) of kas_prefill_index_offsets.
 *     Hs = Hkv, or 1 when desc->pool_scope is 1 (one shared set).
 *   - Selection is exact: the k largest pooled scores, ties to the lower key
 *     index, scores compared as fp32.
 */
#ifndef KASCADE_H
#define KASCADE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KAS_OK = 0,
  KAS_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad shape, bad value */
  KAS_ERR_UNSUPPORTED = 2,        /* valid request the library does not run */
  KAS_ERR_WORKSPACE_TOO_SMALL = 3,
  KAS_ERR_HIP = 4                 /* a HIP launch/runtime call failed */
} kas_status_t;

/* Element type of q, k, v and o. The README's own kernels run fp16 only
 * (README notes); bf16 and fp16 take the same paths here, with 16-bit MFMA of
 * that type, fp32 accumulation and softmax, and probabilities rounded to the
 * element type for P.V. fp32 is decode only. */
typedef enum { KAS_DTYPE_F32 = 0, KAS_DTYPE_BF16 = 1, KAS_DTYPE_F16 = 2 } kas_dtype_t;

typedef enum {
  KAS_OP_DECODE_ANCHOR = 0,
  KAS_OP_DECODE_REUSE = 1,
  KAS_OP_PREFILL_ANCHOR = 2,
  KAS_OP_PREFILL_REUSE = 3,
  KAS_OP_DECODE_DENSE = 4,
  KAS_OP_PREFILL_DENSE = 5
} kas_op_t;

/* Problem description shared by all calls of one layer. */
typedef struct kas_desc {
  int32_t batch;        /* B >= 1 */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads; Hq / Hkv in {1, 2, 4, 8} */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* D in {64, 128} */
  int64_t seq_len;      /* decode: keys in the cache (the new token's key
                           included); prefill: prompt length, a multiple of
                           the tile. N < 2^31. */
  int32_t topk_pct;     /* 1..100: k is this percentage of the candidates
                           (README: "k=10", "--topk 10") */
  int32_t tile;         /* prefill query tile; must be 32 (README notes) */
  int32_t dtype;        /* kas_dtype_t. decode: F32, BF16 or F16; prefill: BF16 or F16 */
  float softmax_scale;  /* <= 0 selects 1/sqrt(head_dim) */
  int64_t kv_batch_stride;  /* elements between batches of k/v; 0 = Hkv*N*D */
  int64_t kv_head_stride;   /* elements between KV heads of k/v; 0 = N*D */
  /* Anchor selection variants (README "Reproducibility": strategies that pool
   * post-softmax scores per KV-head group or over all heads). Zero is the
   * method's own selection. */
  int32_t pool_scope;   /* 0: one index set per KV head, pooled over the
                           Hq/Hkv query heads sharing it (sets [B, Hkv, ..]);
                           1: one set per batch row (decode) or tile
                           (prefill), pooled over all Hq query heads and shared
                           by every KV head (sets [B, 1, ..]); Hq <= 256 */
  int32_t pool_op;      /* 0: pooled score = sum of the heads' (and, in
                           prefill, the tile rows') probabilities; 1: their
                           maximum */
  int32_t query_head_map;  /* reuse calls: 0: head_map has one entry per KV
                              head (all its query heads read that set); 1:
                              one entry per query head (n_q_heads entries,
                              required), each query head gathering its own
                              set's rows (G times the rows of the KV-head
                              map). The README stores head mappings per model
                              ("Running Evaluations"). */
  /* Element strides of q and o (head_dim stays contiguous), so that views
   * such as a [B, N, Hq, D] projection output can be passed without a copy.
   * 0 = the contiguous default: batch Hq*D (decode) or Hq*N*D (prefill), head
   * D (decode) or N*D (prefill), token D (prefill; decode has one token and
   * ignores it). Given values must be positive multiples of 16 bytes; q may
   * alias itself (it is only read), o must not: its rows (b, h, token) may not
   * overlap (KAS_ERR_INVALID_ARGUMENT). */
  int64_t q_batch_stride, q_head_stride, q_token_stride;
  int64_t o_batch_stride, o_head_stride, o_token_stride;
  /* Anchor calls only (others ignore it). 0: the layer's output attends over
   * its own selected set, as a reuse layer with the identity map would (the
   * reading this library takes; the README "Abstract" leaves it open); 1: the
   * output is dense attention over all keys (causal in prefill), computed as
   * kas_decode_dense / kas_prefill_dense compute it, with the sets selected
   * exactly as with 0. For comparisons against schedules whose anchor layers
   * attend densely. */
  int32_t anchor_dense_output;
} kas_desc_t;

/* round-half-up(pct * n / 100) clamped to [0, n]; 0 for n <= 0 or pct <= 0.
 * Host-only, no GPU needed. */
int64_t kas_topk_count(int64_t n_candidates, int32_t pct);

/* Prefill CSR layout: tile t (rows [tile*t, tile*t+tile)) selects
 * kas_topk_count(tile*t, pct) keys among the keys before it, so tile 0
 * selects none. offsets (may be NULL) receives T+1 entries, T = N / tile;
 * *total receives offsets[T]. Host-only. */
kas_status_t kas_prefill_index_offsets(const kas_desc_t* desc, int64_t* offsets, int64_t* total);

/* Device workspace bytes needed by `op` (a kas_op_t) for this description.
 * Host-only. The workspace carries no state between calls. */
kas_status_t kas_workspace_size(const kas_desc_t* desc, int32_t op, size_t* bytes);

/* Decode anchor layer (README "Abstract": exact Top-k in anchor layers).
 * For each (b, KV head g): the logits of the G = Hq/Hkv query heads over all
 * N keys, each head's softmax, the probabilities summed over the G heads
 * (head-aware pooling), the exact Top-kd of that pooled score written to
 * idx_out[b, g, :] ascending, and o[b, h] = attention of head h renormalised
 * over the selected keys. idx_out: [B, Hkv, kd] int32; o: [B, Hq, D].
 * pool_scope 1 pools all Hq heads into one set idx_out[b, 0, :] that every
 * head attends over; pool_op 1 pools by maximum instead of sum. */
kas_status_t kas_decode_anchor(const kas_desc_t* desc, const void* q, const void* k,
                               const void* v, int32_t* idx_out, void* o,
                               void* ws, size_t ws_bytes, void* stream);

/* Decode reuse layer (README "Abstract": indices reused in intermediate
 * layers, head-aware). KV head g attends, for each of its query heads, only
 * over anchor_idx[b, head_map[g], :] (kd keys from the anchor call with the
 * same N and pct) using this layer's own q, k, v.
 * anchor_idx: [B, anchor_kv_heads, kd]; head_map: device int32 [Hkv] with
 * values in [0, anchor_kv_heads) (trusted on the device; NULL = identity,
 * which needs anchor_kv_heads == Hkv, or every KV head reading set 0 when
 * anchor_kv_heads == 1, as for an anchor with pool_scope 1). o: [B, Hq, D]. */
kas_status_t kas_decode_reuse(const kas_desc_t* desc, const void* q, const void* k,
                              const void* v, const int32_t* anchor_idx,
                              int32_t anchor_kv_heads, const int32_t* head_map, void* o,
                              void* ws, size_t ws_bytes, void* stream);

/* Prefill anchor layer (README "Abstract": tile-level operations). For each
 * (b, tile t, KV head g): every query row of the tile and every head of the
 * group gets its causal softmax; the probabilities of keys before the tile
 * are summed over the tile's rows and the group's heads; the exact Top-k_t
 * is tile t's set. Row i of tile t then attends over that set plus its causal
 * diagonal keys [tile*t, i]. idx_out: [B, Hkv, total] CSR; o: [B, Hq, N, D].
 * pool_scope 1 pools the tile's rows of all Hq heads into one set per tile
 * (idx_out [B, 1, total]); pool_op 1 pools by maximum.
 * bf16 or fp16. KAS_ERR_UNSUPPORTED when the index set of one KV head would
 * exceed 2^31 - 1 entries (total; about N > 1.17M at 10 %) or a KV head's
 * slice of k or v reaches 2^31 bytes (N * D * 2). */
kas_status_t kas_prefill_anchor(const kas_desc_t* desc, const void* q, const void* k,
                                const void* v, int32_t* idx_out, void* o,
                                void* ws, size_t ws_bytes, void* stream);

/* Prefill reuse layer: tile t of KV head g attends over the anchor's set of
 * tile t for anchor KV head head_map[g] plus the causal diagonal keys.
 * anchor_idx: [B, anchor_kv_heads, total] CSR from kas_prefill_anchor with the
 * same N, tile and pct; every index of tile t must be < tile*t (trusted on
 * the device). head_map as in kas_decode_reuse. bf16 or fp16. The size limits
 * of kas_prefill_anchor apply. */
kas_status_t kas_prefill_reuse(const kas_desc_t* desc, const void* q, const void* k,
                               const void* v, const int32_t* anchor_idx,
                               int32_t anchor_kv_heads, const int32_t* head_map, void* o,
                               void* ws, size_t ws_bytes, void* stream);

/* Dense baselines. The pages state Kascade's speed-ups against dense
 * attention (README "Abstract": a FlashAttention-3 baseline; its benchmarks
 * run FlashAttention-3 code). These calls compute that dense attention with
 * this library's own kernels, for comparison at the same shapes: the textbook
 * softmax(Q K^T * scale) V ("I/O complexity of attention" abstract).
 * topk_pct is not used (it must still be in range); head_map and index sets
 * do not exist here.
 *
 * Decode: o[b, h] = attention of query head h over all N keys of KV head
 * h / G (split-K over the cache, then a merge of the splits). Layouts as in
 * kas_decode_anchor; any dtype; workspace from
 * kas_workspace_size(KAS_OP_DECODE_DENSE). */
kas_status_t kas_decode_dense(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                              void* o, void* ws, size_t ws_bytes, void* stream);

/* Prefill: causal attention, row i over keys [0, i]. Layouts as in
 * kas_prefill_anchor; bf16 or fp16; N a multiple of the tile (32). Needs no
 * workspace (ws may be NULL; kas_workspace_size(KAS_OP_PREFILL_DENSE) is 0).
 * KAS_ERR_UNSUPPORTED when a KV head's slice of k or v reaches 2^31 bytes. */
kas_status_t kas_prefill_dense(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                               void* o, void* ws, size_t ws_bytes, void* stream);

/* KV caches whose sequences have different lengths and/or whose rows live in
 * pages (README notes: paged and varlen kernels are announced for the pages'
 * own kernels). Passed to the *_kv decode and prefill calls; NULL there means
 * the dense [B, Hkv, N, D] cache of kas_desc_t with every sequence N keys
 * long, exactly the calls without _kv.
 *   - seq_lens (device [B] or NULL): keys of sequence b, in [1, desc->seq_len]
 *     (values outside are clamped into it on the device); the new token's key
 *     is the sequence's last. Sequence b's sets hold max(1,
 *     kas_topk_count(seq_lens[b], pct)) keys; index arrays keep the shape
 *     that desc->seq_len gives, entries past a sequence's count are
 *     unspecified.
 *   - block_table (device [B, max_pages] or NULL for the contiguous cache of
 *     desc): the page holding keys [P i, P i + P) of sequence b. Page ids are
 *     trusted (ids outside [0, num_pages) read page 0). k and v are then page
 *     pools, [num_pages, Hkv, P, D] with the default strides; desc's
 *     kv_*_stride are not used. Paged caches hold bf16 or fp16.
 * KAS_ERR_UNSUPPORTED: a paged fp32 cache, or a pool of 2^31 rows or more
 * (num_pages * page_stride / head_dim). The prefill *_kv calls read lengths
 * in whole tiles (see below). */
typedef struct kas_kv_cache {
  const int32_t* seq_lens;
  const int32_t* block_table;
  int32_t page_size;         /* P: a power of two in [16, 2^20] */
  int32_t max_pages;         /* entries per block_table row, >= ceil(seq_len / P) */
  int64_t num_pages;         /* pages in each of the k and v pools */
  int64_t page_stride;       /* elements between pages, a multiple of head_dim (0 = Hkv * P * D) */
  int64_t page_head_stride;  /* elements between KV heads in a page (0 = P * D) */
} kas_kv_cache_t;

/* Workspace of a *_kv call (any KAS_OP_*): a paged prefill call needs room
 * for contiguous copies of its K and V (2 * B * Hkv * seq_len * head_dim
 * elements) beyond the workspace of the same call without pages. */
kas_status_t kas_workspace_size_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, int32_t op,
                                   size_t* bytes);
/* kas_decode_anchor / kas_decode_reuse / kas_decode_dense over such a cache. */
kas_status_t kas_decode_anchor_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, int32_t* idx_out, void* o, void* ws,
                                  size_t ws_bytes, void* stream);
kas_status_t kas_decode_reuse_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                 const void* k, const void* v, const int32_t* anchor_idx,
                                 int32_t anchor_kv_heads, const int32_t* head_map, void* o, void* ws,
                                 size_t ws_bytes, void* stream);
kas_status_t kas_decode_dense_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                 const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                                 void* stream);

/* The prefill calls over sequences of different lengths: cache->seq_lens
 * (device [B]) gives each prompt's length, taken in whole tiles of 32 rows
 * (clamped to [32, desc->seq_len]); tiles past a prompt are not computed and
 * their rows of o and their index sets are left unspecified. The CSR layout
 * is that of desc->seq_len (a tile's set size depends only on the tile).
 * With block_table, k and v are page pools as for decode (P >= 16, desc->
 * seq_len the longest prompt): the call first copies the K and V rows of
 * every prompt's whole tiles, page by page, into its workspace as a
 * contiguous [B, Hkv, seq_len, D] cache and then runs as over a contiguous
 * one, so its results equal those of the same call on that cache. */
kas_status_t kas_prefill_anchor_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                   const void* k, const void* v, int32_t* idx_out, void* o, void* ws,
                                   size_t ws_bytes, void* stream);
kas_status_t kas_prefill_reuse_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, const int32_t* anchor_idx,
                                  int32_t anchor_kv_heads, const int32_t* head_map, void* o, void* ws,
                                  size_t ws_bytes, void* stream);
kas_status_t kas_prefill_dense_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, void* o, void* ws, size_t ws_bytes,
                                  void* stream);

/* kas_decode_reuse for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same call and results, with the split-K partials in a static device
 * buffer of the library (KAS_NOALLOC_SCRATCH_BYTES per GPU, held until the
 * process ends) instead of a caller workspace. Calls needing more scratch
 * than that (kas_workspace_size(KAS_OP_DECODE_REUSE) of the same descriptor)
 * return KAS_ERR_UNSUPPORTED and enqueue nothing. The current device must be
 * the stream's device. Every call on one GPU shares that GPU's buffer: calls
 * that overlap in time on one GPU (other streams, other threads) race and
 * must be serialised by the caller. Nothing in it needs to start at zero. */
#define KAS_NOALLOC_SCRATCH_BYTES (16u << 20)
kas_status_t kas_decode_reuse_noalloc(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                                      const int32_t* anchor_idx, int32_t anchor_kv_heads, const int32_t* head_map,
                                      void* o, void* stream);

/* Refined layer of proposal-refined reuse (decode). The Prism Attention page
 * (thelatestinai.com/papers/2610.22985, "Proposal-Refined" sharing) has a
 * proposal layer export a pool of rho * kappa candidate keys and every
 * refined layer select its own kappa keys within that pool; here the pool is
 * an anchor call's index set at a larger percentage (rho times the layer's)
 * and kappa is this layer's own max(1, kas_topk_count(N, pct)). For each
 * (b, KV head g): pool = pool_idx[b, head_map[g], :pool_size] (ascending
 * keys); each query head's softmax over the pool's keys with this layer's
 * q and K, summed over the group's heads; the exact Top-kappa within the pool
 * (ties to the lower key) written to idx_out[b, g, :kappa] ascending; each
 * head attends over it. pool_idx [B, pool_kv_heads, pool_size], kappa <=
 * pool_size <= N; head_map as in kas_decode_reuse (values in [0,
 * pool_kv_heads)); idx_out [B, Hkv, kappa]; o [B, Hq, D]. pool_scope and
 * pool_op must be 0 (KAS_ERR_UNSUPPORTED). With query_head_map = 1 every
 * query head h is a set of its own: its pool is pool_idx[b, head_map[h], :]
 * (head_map of Hq entries, required), it selects its Top-kappa by its own
 * softmax over the pool, and idx_out is [B, Hq, kappa]. */
kas_status_t kas_workspace_size_refine(const kas_desc_t* desc, int64_t pool_size, size_t* bytes);
kas_status_t kas_decode_refine(const kas_desc_t* desc, const void* q, const void* k, const void* v,
                               const int32_t* pool_idx, int32_t pool_kv_heads, int64_t pool_size,
                               const int32_t* head_map, int32_t* idx_out, void* o, void* ws,
                               size_t ws_bytes, void* stream);
/* The same over a cache described by a kas_kv_cache_t; a NULL cache and NULL
 * pool_lens give exactly kas_decode_refine. With cache->block_table the
 * pool's keys are translated to rows of the page pools before scoring, and
 * the refined keys again before the attention; the results equal those of a
 * contiguous cache. Sequences of different lengths (cache->seq_lens, L_b
 * clamped to [1, seq_len]) and pools of different sizes (pool_lens: device
 * [B] or NULL, the valid entries of sequence b's pool rows, e.g. max(1,
 * kas_topk_count(L_b, pct_pool)) after an anchor call over the same cache):
 * sequence b refines within its first pool_b = clamp(pool_lens[b] (or
 * pool_size), 1, min(pool_size, L_b)) pool entries and keeps kappa_b =
 * min(max(1, kas_topk_count(L_b, pct)), pool_b) keys, which is what the call
 * on that sequence alone (seq_len L_b, pool_size pool_b) computes. Entries of
 * idx_out past kappa_b are unspecified. Pool entries are trusted to be keys
 * of the sequence (keys outside [0, seq_len) read key 0). */
kas_status_t kas_workspace_size_refine_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, int64_t pool_size,
                                          size_t* bytes);
kas_status_t kas_decode_refine_kv(const kas_desc_t* desc, const kas_kv_cache_t* cache, const void* q,
                                  const void* k, const void* v, const int32_t* pool_idx, int32_t pool_kv_heads,
                                  int64_t pool_size, const int32_t* pool_lens, const int32_t* head_map,
                                  int32_t* idx_out, void* o, void* ws, size_t ws_bytes, void* stream);

/* Process-wide tuning options. They select alternative but equivalent code
 * paths (every setting gives the same results) and the sizes of internal
 * buffers; tests use them to reach the alternative paths, benchmarks to
 * compare them. Settings apply to calls (and workspace-size queries) made
 * after them, in any thread; a value of -1 restores the default. Not meant
 * to change while another thread is between kas_workspace_size and the call
 * it sized. */
typedef enum {
  KAS_OPT_DECODE_SPLIT_ROWS = 0,    /* index-set rows per decode gather workgroup, 16..2048
                                       (default -1: sized so one wave of workgroups covers the chip) */
  KAS_OPT_DECODE_SELECT_ONE_PASS = 1, /* 1: decode Top-k by one workgroup per index set (one launch);
                                         0: spread over the chip in three launches; default -1: one
                                         workgroup per set for sets of at most 8192 keys, else spread */
  KAS_OPT_PREFILL_POOL_MB = 2,      /* cap of the prefill pooled-score buffer, MiB (default 16384);
                                       longer prompts run their pooling and selection in tile ranges */
  KAS_OPT_PREFILL_SELECT_CAP = 3,   /* 0..8192 (default 8192): the largest first-digit bin the prefill
                                       Top-k resolves in LDS; larger bins take in-place passes */
  KAS_OPT_COUNT_ = 4
} kas_option_t;
/* KAS_ERR_INVALID_ARGUMENT for an unknown option or a value out of range. */
kas_status_t kas_set_option(int32_t option, int64_t value);
kas_status_t kas_get_option(int32_t option, int64_t* value);

/* Text of a status code; any int (also values outside kas_status_t) is accepted. */
const char* kas_status_string(int32_t status);
/* Text of the last failure on the calling thread ("" if none). */
const char* kas_last_error(void);

/* Optional kernel timing (for benchmarks). While enabled, every kernel the
 * library launches is bracketed by HIP events on its stream. kas_profile_query
 * waits for the recorded events and returns the summed device time (ms) and
 * launch count of kernels whose name equals `kernel`; kas_profile_names writes
 * the known kernel names, comma separated. Not thread-safe against concurrent
 * calls that launch work. */
kas_status_t kas_profile_enable(int32_t enable);
kas_status_t kas_profile_reset(void);
kas_status_t kas_profile_query(const char* kernel, double* total_ms, int64_t* launches);
kas_status_t kas_profile_names(char* buf, size_t buf_len);

#ifdef __cplusplus
}
#endif
#endif /* KASCADE_H */
