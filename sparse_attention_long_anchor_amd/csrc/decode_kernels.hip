// Decode-phase kernels for gfx950 (one new query token per sequence).
//
//  dec_score    anchor: stream the K cache once, logits of the G query heads
//               of each KV head on a 16x16 MFMA tile, base-2 logits to the
//               workspace, per-chunk softmax statistics (max, sum of exp).
//  dec_pool     anchor: global softmax statistics per head, pooled score
//               P_j = sum over the group's heads of the post-softmax
//               probability (Kascade README "Abstract": exact post-softmax
//               Top-k, head-aware), first radix digit histogram.
//  sel_*        anchor: exact k-th largest pooled score by a three-digit
//               radix select over the fp32 bit pattern (candidates of the
//               first digit's bin per chunk, digits 2 and 3 resolved per row),
//               then a stable compaction of {P > tau} plus the lowest-index
//               ties.
//  dec_attn     anchor and reuse: index-driven gather of K/V rows, online
//               softmax, split-K partial (o, m, l) per workgroup.
//  dec_combine  merge of the split-K partials into the output.
#include "kas_device.hpp"
#include <stdlib.h>

#include <string.h>
#include <type_traits>

#include "kas_block.hpp"
#include "kas_internal.hpp"

namespace kas {

constexpr int kMaxSplitRows = 2048;

// KV head of workgroup head index g: g itself, or with one anchor set per
// query head (the reuse kernels then run one query head per "KV head", G = 1)
// the query head's KV head g / kvdiv.
__device__ __forceinline__ int kv_head(const DecodeArgs& a, int g) { return a.kvdiv > 1 ? g / a.kvdiv : g; }

// Keys of sequence b (all sequences have N unless lengths are given).
// (lengths are trusted inputs, clamped to [1, N])
__device__ __forceinline__ int64_t seq_n(const DecodeArgs& a, int b) {
  if (!a.seq_lens) return a.N;
  const int64_t n = a.seq_lens[b];
  return n < 1 ? 1 : (n > a.N ? a.N : n);
}
// Rows of sequence b's sets in a gather: its k, or (dense) all its keys.
__device__ __forceinline__ int64_t set_rows(const DecodeArgs& a, int b) {
  if (a.set_lens) return a.set_lens[b];
  if (!a.seq_lens) return a.kk;
  const int64_t n = seq_n(a, b);
  return a.rows_are_keys ? n : decode_k_of(n, a.pct);
}
// Keys the selection keeps for one of its units (sets).
__device__ __forceinline__ uint32_t unit_k(const DecodeArgs& a, int64_t unit) {
  const int64_t per_b = a.sel_units / a.B;
  if (a.set_lens) return (uint32_t)a.set_lens[unit / per_b];
  if (!a.seq_lens) return (uint32_t)a.kk;
  return (uint32_t)decode_k_of(seq_n(a, (int)(unit / per_b)), a.pct);
}
// A page id from the block table (trusted input, clamped to the pool).
__device__ __forceinline__ int64_t page_id(const DecodeArgs& a, int32_t p) {
  return ((uint64_t)p < (uint64_t)a.num_pages) ? p : 0;
}

constexpr int kScorePages = kScoreMaxRows / 16 + 1;  // pages a scoring chunk can touch

// ------------------------------------------------------------------ dec_score

constexpr float kBigSum = 0x1p64f;   // lazy-reference term that forces the exact update

// PG: a paged cache; the chunk's page ids are read into LDS once, and a
// 16-key block (pages hold a power-of-two multiple of 16 keys) lies in one page.
// IX: rows are the keys of a pool (a.idx through the head map, a.N = pool
// size); the chunk's keys are read into LDS once. IX with PG: the pool's keys
// are physical rows of a page pool (translated beforehand), counted in D
// elements from k + g * page_hstride.
//
// 16-bit rows are loaded whole (each load instruction reads 64 / (D / 8)
// complete rows, non-temporally except for pool rows, which neighbouring
// chunks share) and re-laid out into the MFMA operand layout through a
// wave-private LDS slot (16-byte chunks XOR-swizzled by row, so both the
// row-wise writes and the operand reads are free of bank conflicts): a
// probe streaming 1 GiB of 256-byte rows in 16-row blocks reached 7.0 TB/s
// this way against 6.2 TB/s with each instruction reading 64 bytes of 16 rows.
template <typename T, int D, int G, bool PG = false, bool IX = false>
__global__ __launch_bounds__(256, 4) void dec_score_kernel(DecodeArgs a) {
  using QK = QKMfma<T, D>;
  constexpr bool ROWS = sizeof(T) == 2;                  // whole-row loads through LDS
  constexpr int ROWB = D * (int)sizeof(T);               // bytes per row
  constexpr int CH = ROWB / 16;                          // 16-byte chunks per row
  constexpr int RPI = 64 / CH;                           // rows per load instruction
  constexpr int NLI = ROWS ? 16 / RPI : 1;               // load instructions per 16-row block
  __shared__ float s_m[4][G], s_l[4][G];
  __shared__ int32_t s_pg[IX ? kScoreMaxRows : (PG ? kScorePages : 1)];
  __shared__ __align__(16) char s_rows[ROWS ? 4 : 1][ROWS ? 16 * ROWB : 16];   // one block per wave
  const int chunk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int64_t row0 = (int64_t)chunk * a.score_rows;
  const int nrows = (int)min((int64_t)a.score_rows, seq_n(a, b) - row0);   // <= 0: nothing to score
  const int64_t unit = (int64_t)b * a.Hkv + g;

  if (chunk == 0) {
    uint32_t* h = a.hist + unit * kHistWords;
    for (int i = tid; i < kHistWords; i += 256) h[i] = 0u;
  }
  const int gk = kv_head(a, g);     // K head of the set (a query head's with one set per query head)
  const T* kb = (const T*)a.k + b * a.kv_bstride + gk * a.kv_hstride + row0 * D;
  const int64_t p0 = row0 >> a.page_shift;
  if (PG && !IX) {
    const int np = nrows > 0 ? (int)(((row0 + nrows - 1) >> a.page_shift) - p0 + 1) : 0;
    for (int i = tid; i < np; i += 256) s_pg[i] = a.block_table[(int64_t)b * a.max_pages + p0 + i];
    __syncthreads();
  }
  if (IX) {
    int ga = a.head_map ? a.head_map[g] : g;
    ga = ((unsigned)ga < (unsigned)a.Hkv_a) ? ga : 0;
    const int32_t* pool = a.idx + ((int64_t)b * a.Hkv_a + ga) * a.N + row0;
    for (int i = tid; i < nrows; i += 256) {
      const int32_t j = pool[i];
      s_pg[i] = ((uint32_t)j < (uint64_t)a.n_keys) ? j : 0;     // trusted input, kept in the cache
    }
    __syncthreads();
  }
  typename QK::QFrag qf;
  QK::load_q(qf, (const T*)a.q + b * a.q_bstride + (int64_t)(g * G + min(c16, G - 1)) * a.q_hstride, c16 < G, q4);
  float* lg = a.logits + (unit * a.N + row0) * G;

  float ml[4], ls[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { ml[r] = kNegInf; ls[r] = 0.f; }

  const int nblk = (nrows + 15) >> 4;
  // Wave w takes 16-row blocks w, w+4, ...; the rows of its next two blocks
  // are in flight in two register sets named at compile time (a runtime
  // swap would copy registers whose loads are still in flight, which waits
  // for them).
  // first element of row jr of the chunk (rows past the chunk read its row 0)
  auto row_ptr = [&](int jr) __attribute__((always_inline)) -> const T* {
    if (IX) {
      const int64_t key = s_pg[jr < nrows ? jr : 0];
      const T* base = PG ? (const T*)a.k + gk * a.page_hstride : (const T*)a.k + b * a.kv_bstride + gk * a.kv_hstride;
      return base + key * D;
    } else if (PG) {
      const int64_t j = row0 + (jr < nrows ? jr : 0);
      const int64_t pg = page_id(a, s_pg[(j >> a.page_shift) - p0]);
      return (const T*)a.k + pg * a.page_stride + gk * a.page_hstride + (j & ((1 << a.page_shift) - 1)) * D;
    } else {
      return kb + (int64_t)(jr < nrows ? jr : 0) * D;
    }
  };
  // the 16 rows of a block: whole rows (16-bit types) or the MFMA operand
  // layout straight from memory (fp32)
  struct Rows { u32x4 r[NLI]; };
  using Buf = typename std::conditional<ROWS, Rows, QK>::type;
  auto load = [&](int blk, Buf& dst) __attribute__((always_inline)) {
    if constexpr (ROWS) {
#pragma unroll
      for (int i = 0; i < NLI; ++i) {
        const T* p = row_ptr(blk * 16 + RPI * i + lane / CH) + 8 * (lane % CH);
        dst.r[i] = IX ? ldg16(p) : ldg16_nt(p);
      }
    } else {
      dst.load_k(row_ptr(blk * 16 + c16), q4);
    }
  };
  // whole rows -> MFMA operand (chunk 4 c + q4 of row c16 for instruction c).
  // One LDS slot per wave serves every block: a wave's LDS accesses execute
  // in order, so a block's rows are written only after the last block's
  // operand reads.
  auto operand = [&](const Buf& src) __attribute__((always_inline)) -> QK {
    if constexpr (ROWS) {
      char* sl = s_rows[wave];
#pragma unroll
      for (int i = 0; i < NLI; ++i) {
        const int row = RPI * i + lane / CH, ch = lane % CH;
        *reinterpret_cast<u32x4*>(sl + row * ROWB + 16 * (ch ^ (row & (CH - 1)))) = src.r[i];
      }
      wave_lds_fence();
      QK kq;
#pragma unroll
      for (int c = 0; c < QK::NI; ++c)
        kq.kf[c] = *reinterpret_cast<const u32x4*>(sl + c16 * ROWB + 16 * ((4 * c + q4) ^ (c16 & (CH - 1))));
      return kq;
    } else {
      return src;
    }
  };
  // STEADY: a full block inside the steady loop (all rows valid); for G = 4
  // and 8 the logits are transposed across lanes so that the whole wave
  // writes them with one unconditional contiguous store (a branch around a
  // store would make the waits before the next block's MFMA drain the loads
  // in flight: stores count on the same counter).
  auto process = [&](int blk, const Buf& buf, auto steady_tag) __attribute__((always_inline)) {
    constexpr bool STEADY = decltype(steady_tag)::value;
    const int jr = blk * 16 + c16;
    const bool val = STEADY || jr < nrows;
    const f32x4 s = operand(buf).run(qf);
    float t[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = val ? s[r] * a.scale_log2 : kNegInf;
    if (STEADY && G == 4) {
      // lane l: key l / 4, head l % 4, held by lane l / 4 in reg l % 4
      const int src_lane = lane >> 2, h = lane & 3;
      float v0 = __shfl(t[0], src_lane), v1 = __shfl(t[1], src_lane);
      float v2 = __shfl(t[2], src_lane), v3 = __shfl(t[3], src_lane);
      asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));   // all four, no branches
      const float v = (h & 2) ? ((h & 1) ? v3 : v2) : ((h & 1) ? v1 : v0);
      lg[(int64_t)blk * 16 * G + lane] = v;
    } else if (STEADY && G == 8) {
      // lane l: key l / 4, heads 2 (l % 4) and +1, held by lane key + 16 q4
      const int h0 = 2 * (lane & 3);
      const int src_lane = (lane >> 2) + 16 * (h0 >> 2);
      float v0 = __shfl(t[0], src_lane), v1 = __shfl(t[1], src_lane);
      float v2 = __shfl(t[2], src_lane), v3 = __shfl(t[3], src_lane);
      asm volatile("" : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(v3));
      const bool lo = (h0 & 3) == 0;
      *reinterpret_cast<float2*>(lg + (int64_t)blk * 16 * G + 2 * lane) =
          lo ? float2{v0, v1} : float2{v2, v3};
    } else if (val && 4 * q4 < G) {
      // lane (key jr, quarter q4) holds heads 4 q4 .. 4 q4 + 3
      float* dst = lg + (int64_t)jr * G + 4 * q4;
      if (G >= 4) {
        *reinterpret_cast<f32x4*>(dst) = f32x4{t[0], t[1], t[2], t[3]};
      } else {
#pragma unroll
        for (int r = 0; r < G; ++r) dst[r] = t[r];
      }
    }
    // Row sums against a lazy per-lane reference: ml is the lane's running
    // offset, and a score is added as exp2(t - ml) without a block maximum.
    // Only a term that is not finite or above 2^64 (the lane's first value,
    // or a score 64 above the reference) sends the wave through the exact
    // update, which moves the reference to the larger of the two.
    float p[4];
    bool over = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = exp2_fast(t[r] - ml[r]);
      over |= !(p[r] <= kBigSum);
    }
    if (__builtin_expect(__any(over), 0)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mn = fmaxf(ml[r], t[r]);
        ls[r] = (ml[r] == kNegInf) ? 0.f : ls[r] * exp2_fast(ml[r] - mn);
        p[r] = (t[r] == kNegInf) ? 0.f : exp2_fast(t[r] - mn);
        ml[r] = mn;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) ls[r] += p[r];
  };
  Buf qa, qb;
  int blk = wave;
  using Steady = std::true_type;
  using Edge = std::false_type;
  if (blk + 12 < nblk) {
    // steady state without a branch around a load (waits stay partial); the
    // entry issues the same loads in the same order as the loop's back edge
    load(blk, qa);
    load(blk + 4, qb);
    for (; blk + 12 < nblk; blk += 8) {     // blocks blk .. blk + 12 all full
      process(blk, qa, Steady{});
      load(blk + 8, qa);
      process(blk + 4, qb, Steady{});
      load(blk + 12, qb);
    }
  } else {
    if (blk < nblk) load(blk, qa);
    if (blk + 4 < nblk) load(blk + 4, qb);
  }
  if (blk < nblk) process(blk, qa, Edge{});
  if (blk + 8 < nblk) load(blk + 8, qa);
  if (blk + 4 < nblk) process(blk + 4, qb, Edge{});
  if (blk + 8 < nblk) process(blk + 8, qa, Edge{});
  // merge the lanes' (reference, sum) pairs of each head: lanes 16 (h / 4) ..
  // + 15 hold head h in register h % 4
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = ml[h & 3];
    const float rowmax = row16_max(m);
    const float lsum = row16_sum(m == kNegInf ? 0.f : ls[h & 3] * exp2_fast(m - rowmax));
    float M = readlane_f(rowmax, 16 * (h >> 2));
    float L = readlane_f(lsum, 16 * (h >> 2));
    if (lane == 0) { s_m[wave][h] = M; s_l[wave][h] = L; }
  }
  __syncthreads();
  if (tid < G) {
    const int h = tid;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += (s_m[w][h] == kNegInf) ? 0.f : s_l[w][h] * exp2_fast(s_m[w][h] - M);
    float* st = a.stats + ((unit * a.n_score_chunks + chunk) * G + h) * 2;
    st[0] = M;
    st[1] = L;
  }
}

// ------------------------------------------------------------------ dec_pool

// One workgroup per (4096-key chunk, set): each head's softmax statistics
// from the score pass's per-chunk (max, sum) pairs, then per key the heads'
// probabilities pooled (OP 0: sum, OP 1: max) and the first-digit histogram
// of the pooled scores. A set is one (b, KV head) over its G query heads, or
// (ALL) one b over all Hkv * G heads.
template <int G, int OP, bool ALL>
__global__ __launch_bounds__(256) void dec_pool_kernel(DecodeArgs a) {
  constexpr int NS = ALL ? kMaxPoolHeads : G;
  __shared__ uint32_t s_hist[kBins1];
  __shared__ float s_tmp[4];
  __shared__ float s_M[NS], s_iL[NS];
  const int chunk = blockIdx.x, b = blockIdx.z;
  const int g0 = ALL ? 0 : blockIdx.y;
  const int nh = ALL ? a.Hkv * G : G;                         // heads pooled into the set
  const int64_t unit = ALL ? b : (int64_t)b * a.Hkv + g0;     // set: pooled row, histogram
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kBins1; i += 256) s_hist[i] = 0u;

  if (!ALL) {
    // the G heads' statistics in one sweep over the chunks (per head the same
    // arithmetic and reduction order as block_max_256 / block_sum_256)
    __shared__ float s_red[4][G];
    const float* st = a.stats + unit * a.n_score_chunks * G * 2;
    float m[G];
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = kNegInf;
    for (int c = tid; c < a.n_score_chunks; c += 256)
#pragma unroll
      for (int h = 0; h < G; ++h) m[h] = fmaxf(m[h], st[(c * G + h) * 2]);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = wave_max(m[h]);
      if (lane == 0) s_red[wave][h] = m[h];
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = fmaxf(fmaxf(s_red[0][h], s_red[1][h]), fmaxf(s_red[2][h], s_red[3][h]));
    float l[G];
#pragma unroll
    for (int h = 0; h < G; ++h) l[h] = 0.f;
    for (int c = tid; c < a.n_score_chunks; c += 256)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mc = st[(c * G + h) * 2];
        l[h] += (mc == kNegInf) ? 0.f : st[(c * G + h) * 2 + 1] * exp2_fast(mc - m[h]);
      }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      l[h] = wave_sum(l[h]);
      if (lane == 0) s_red[wave][h] = l[h];
    }
    __syncthreads();
    if (tid < G) {
      const int h = tid;
      s_M[h] = m[h];
      s_iL[h] = 1.0f / ((s_red[0][h] + s_red[1][h]) + (s_red[2][h] + s_red[3][h]));
    }
  } else {
    // head x of the set is query head r = x % G of KV head g0 + x / G
    for (int x = 0; x < nh; ++x) {
      const int64_t ug = (int64_t)b * a.Hkv + g0 + x / G;
      const int h = x % G;
      const float* st = a.stats + ug * a.n_score_chunks * G * 2;
      float m = kNegInf;
      for (int c = tid; c < a.n_score_chunks; c += 256) m = fmaxf(m, st[(c * G + h) * 2]);
      const float M = block_max_256(m, s_tmp);
      float l = 0.f;
      for (int c = tid; c < a.n_score_chunks; c += 256) {
        float mc = st[(c * G + h) * 2];
        l += (mc == kNegInf) ? 0.f : st[(c * G + h) * 2 + 1] * exp2_fast(mc - M);
      }
      const float L = block_sum_256(l, s_tmp);
      if (tid == 0) { s_M[x] = M; s_iL[x] = 1.0f / L; }
    }
  }
  __syncthreads();
  auto pool = [](float acc, float p) __attribute__((always_inline)) { return OP ? fmaxf(acc, p) : acc + p; };

  float* P = a.pooled + unit * a.pstride;
  const int64_t base = (int64_t)chunk * kSelChunk;
  const int64_t Nb = seq_n(a, b);       // keys past the sequence's end pool to 0
  if (!ALL) {
    float M[G], iL[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { M[h] = s_M[h]; iL[h] = s_iL[h]; }
    const float* lg = a.logits + unit * a.N * G;
#pragma unroll 4
    for (int i = 0; i < kSelChunk / 256; ++i) {
      const int64_t j = base + i * 256 + tid;
      if (j < a.N) {
        float acc = 0.f;
        if (j < Nb) {
          if constexpr (G % 4 == 0) {
            // the key's G logits in 16-byte loads
#pragma unroll
            for (int h4 = 0; h4 < G; h4 += 4) {
              const f32x4 t4 = *reinterpret_cast<const f32x4*>(lg + j * G + h4);
#pragma unroll
              for (int e = 0; e < 4; ++e) acc = pool(acc, exp2_fast(t4[e] - M[h4 + e]) * iL[h4 + e]);
            }
          } else {
#pragma unroll
            for (int h = 0; h < G; ++h) acc = pool(acc, exp2_fast(lg[j * G + h] - M[h]) * iL[h]);
          }
        }
        P[j] = acc;
        atomicAdd(&s_hist[__float_as_uint(acc) >> 21], 1u);
      }
    }
  } else {
    // heads in KV-head order, each KV head's G logits of a key contiguous
    const int64_t gstride = a.N * G;
    const float* lg0 = a.logits + (int64_t)b * a.Hkv * gstride;
    for (int i = 0; i < kSelChunk / 256; ++i) {
      const int64_t j = base + i * 256 + tid;
      if (j < a.N) {
        float acc = 0.f;
        for (int g = 0; g < (j < Nb ? a.Hkv : 0); ++g) {
          const float* lg = lg0 + g * gstride + j * G;
#pragma unroll
          for (int h = 0; h < G; ++h) acc = pool(acc, exp2_fast(lg[h] - s_M[g * G + h]) * s_iL[g * G + h]);
        }
        P[j] = acc;
        atomicAdd(&s_hist[__float_as_uint(acc) >> 21], 1u);
      }
    }
  }
  __syncthreads();
  uint32_t* gh = a.hist + unit * kHistWords;
  for (int i = tid; i < kBins1; i += 256)
    if (s_hist[i]) atomicAdd(&gh[i], s_hist[i]);
}

// ------------------------------------------------------------------ radix select

// Chunked selection, step 1 (one workgroup per 4096-score chunk): the bin b1
// of the k-th largest from the first-digit histogram; the chunk's count of
// scores in higher bins (all of them are kept) and its scores of bin b1, in
// position order, in the chunk's own slot of the candidate area. The chunk's
// loads are issued before the bin search so the two latencies overlap.
__global__ __launch_bounds__(256) void sel_cand_kernel(DecodeArgs a) {
  __shared__ uint32_t s_tmp[4];
  __shared__ int s_res[2];
  const int chunk = blockIdx.x;
  const int64_t unit = blockIdx.y;
  const int tid = threadIdx.x;
  const uint32_t* P = reinterpret_cast<const uint32_t*>(a.pooled + unit * a.pstride);
  constexpr int PER = kSelChunk / 256;
  const int64_t j0 = (int64_t)chunk * kSelChunk + tid * PER;
  uint32_t u[PER];
  if (j0 + PER <= a.N) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const u32x4 v = ldg16(P + j0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * q + e] = v[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) u[i] = (j0 + i < a.N) ? P[j0 + i] : 0u;
  }
  int b1;
  uint32_t ab1;
  block_find_bin(a.hist + unit * kHistWords, kBins1, unit_k(a, unit), s_tmp, s_res, b1, ab1);
  uint32_t gt = 0, nc = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool in = j0 + i < a.N;
    gt += (in && (u[i] >> 21) > (uint32_t)b1) ? 1u : 0u;
    nc += (in && (u[i] >> 21) == (uint32_t)b1) ? 1u : 0u;
  }
  // both counts fit 16 bits (at most kSelChunk per chunk): one packed scan
  uint32_t tot;
  const uint32_t ex = block_excl_scan_256((gt << 16) | nc, s_tmp, &tot);
  uint32_t pos = ex & 0xffffu;
  uint32_t* cand = a.cand + (unit * a.n_sel_chunks + chunk) * (int64_t)kSelChunk;
#pragma unroll
  for (int i = 0; i < PER; ++i)
    if (j0 + i < a.N && (u[i] >> 21) == (uint32_t)b1) cand[pos++] = u[i];
  if (tid == 0) {
    uint32_t* c = a.counts + (unit * a.n_sel_chunks + chunk) * 2;
    c[0] = tot >> 16;
    c[1] = tot & 0xffffu;
  }
}

// Chunked selection, step 3: stable compaction. Key j is kept if P_j > tau,
// or P_j == tau and fewer than r equal keys precede it; output position = kept
// keys before j (the chunk's prefix counts from step 2 plus a workgroup scan).
__global__ __launch_bounds__(256) void sel_compact_kernel(DecodeArgs a) {
  __shared__ uint32_t s_tmp[4];
  const int chunk = blockIdx.x;
  const int64_t unit = blockIdx.y;
  const int tid = threadIdx.x;
  const uint32_t tau = a.selstate[unit * 4 + 0];
  const uint32_t r = a.selstate[unit * 4 + 1];
  // scores above / equal to tau in the chunks before this one
  const uint32_t* c = a.counts + (unit * a.n_sel_chunks + chunk) * 2;
  const uint32_t gt_before = c[0], eq_before = c[1];
  const uint32_t* P = reinterpret_cast<const uint32_t*>(a.pooled + unit * a.pstride);
  // thread owns 16 consecutive keys (16-byte loads inside the row)
  constexpr int PER = kSelChunk / 256;
  const int64_t j0 = (int64_t)chunk * kSelChunk + tid * PER;
  uint32_t u[PER];
  if (j0 + PER <= a.N) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const u32x4 v = ldg16(P + j0 + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * q + e] = v[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) u[i] = (j0 + i < a.N) ? P[j0 + i] : 0u;
  }
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool in = j0 + i < a.N;
    gt += (in && u[i] > tau) ? 1u : 0u;
    eq += (in && u[i] == tau) ? 1u : 0u;
  }
  // both counts fit 16 bits (at most kSelChunk per chunk): one packed scan
  const uint32_t ex = block_excl_scan_256((gt << 16) | eq, s_tmp, nullptr);
  uint32_t g_ex = (ex >> 16) + gt_before;
  uint32_t e_ex = (ex & 0xffffu) + eq_before;
  int32_t* out = a.idx_out + unit * a.kk;
  const uint32_t ku = unit_k(a, unit);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if (j0 + i >= a.N) break;
    if (u[i] > tau) {
      const uint32_t pos = g_ex + min(e_ex, r);
      if (pos < ku) out[pos] = (int32_t)(j0 + i);
      ++g_ex;
    } else if (u[i] == tau) {
      if (e_ex < r && g_ex + e_ex < ku) out[g_ex + e_ex] = (int32_t)(j0 + i);
      ++e_ex;
    }
  }
}

// One workgroup of 1024 threads per (b, g) finishes the radix select whose
// first digit (bits 31..21) dec_pool histogrammed:
//  1. the bin b1 of the k-th largest; its population is known from the
//     histogram, so if it fits, one sweep of the pooled row collects the bin's
//     scores into LDS and digits 2 (bits 20..10) and 3 (bits 9..0) are
//     resolved there; otherwise two more sweeps histogram them in place;
//  2. tau (the exact bit pattern of the k-th largest) and r (how many scores
//     equal to tau are kept);
//  3. a last sweep writes every key with P > tau plus the first r keys equal
//     to tau, in index order (one packed workgroup scan per step).
// Sweeps read 16 consecutive scores per thread per step with the next step's
// loads already in flight (32 scores per thread in registers).
constexpr int kSelThreads = 1024;
constexpr int kSelCandCap = 24576;   // LDS candidate list (96 KB)
__global__ __launch_bounds__(kSelThreads) void sel_fused_kernel(DecodeArgs a) {
  __shared__ uint32_t s_h[kBins2];
  __shared__ uint32_t s_cand[kSelCandCap];
  __shared__ uint32_t s_tmp[kSelThreads / 64];
  __shared__ int s_res[2];
  __shared__ uint32_t s_ncand;
  const int64_t unit = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t k = unit_k(a, unit);
  const uint32_t* P = reinterpret_cast<const uint32_t*>(a.pooled + unit * a.pstride);
  const uint32_t* hist1 = a.hist + unit * kHistWords;
  const int64_t N = a.N;
  constexpr int PER = 16;
  constexpr int64_t STEP = (int64_t)kSelThreads * PER;
  int b1, b2, b3;
  uint32_t ab1, ab2, ab3;
  block_find_bin_nt<kSelThreads>(hist1, kBins1, k, s_tmp, s_res, b1, ab1);
  const uint32_t nb1 = hist1[b1];
  for (int i = tid; i < kBins2; i += kSelThreads) s_h[i] = 0u;
  if (tid == 0) s_ncand = 0u;
  __syncthreads();

  // 16 scores of this thread at base + 16 tid (positions >= N read as 0 and
  // are excluded by the callers through the position test)
  auto load16 = [&](int64_t base, uint32_t* u) __attribute__((always_inline)) {
    const int64_t j0 = base + (int64_t)tid * PER;
    if (j0 + PER <= N) {
#pragma unroll
      for (int q = 0; q < PER / 4; ++q) {
        const u32x4 v = ldg16(P + j0 + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) u[4 * q + e] = v[e];
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) u[i] = (j0 + i < N) ? P[j0 + i] : 0u;
    }
  };
  // sweep with the next step's loads in flight; fn(base, u) per step
  auto sweep = [&](auto&& fn) __attribute__((always_inline)) {
    uint32_t ua[PER], ub[PER];
    load16(0, ua);
    for (int64_t base = 0; base < N; base += 2 * STEP) {
      if (base + STEP < N) load16(base + STEP, ub);
      fn(base, ua);
      if (base + 2 * STEP < N) load16(base + 2 * STEP, ua);
      if (base + STEP < N) fn(base + STEP, ub);
    }
  };

  if (nb1 <= (uint32_t)kSelCandCap) {
    // collect bin b1 into LDS (wave-aggregated appends)
    sweep([&](int64_t base, const uint32_t* u) __attribute__((always_inline)) {
      const int64_t j0 = base + (int64_t)tid * PER;
      uint32_t c = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) c += (j0 + i < N && (u[i] >> 21) == (uint32_t)b1) ? 1u : 0u;
      const uint32_t inc = wave_incl_scan_u32(c);
      uint32_t wbase = 0;
      if (lane == 63 && inc) wbase = atomicAdd(&s_ncand, inc);
      wbase = __shfl(wbase, 63);
      uint32_t pos = wbase + inc - c;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (j0 + i < N && (u[i] >> 21) == (uint32_t)b1) {
          if (pos < (uint32_t)kSelCandCap) s_cand[pos] = u[i];
          ++pos;
        }
      }
    });
    __syncthreads();
    const uint32_t nc = min(s_ncand, (uint32_t)kSelCandCap);
    for (uint32_t i = tid; i < nc; i += kSelThreads) atomicAdd(&s_h[(s_cand[i] >> 10) & 0x7ffu], 1u);
    __syncthreads();
    block_find_bin_nt<kSelThreads>(s_h, kBins2, k - ab1, s_tmp, s_res, b2, ab2);
    for (int i = tid; i < kBins3; i += kSelThreads) s_h[i] = 0u;
    __syncthreads();
    const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
    for (uint32_t i = tid; i < nc; i += kSelThreads)
      if ((s_cand[i] >> 10) == pre) atomicAdd(&s_h[s_cand[i] & 0x3ffu], 1u);
    __syncthreads();
    block_find_bin_nt<kSelThreads>(s_h, kBins3, k - ab1 - ab2, s_tmp, s_res, b3, ab3);
  } else {
    sweep([&](int64_t base, const uint32_t* u) __attribute__((always_inline)) {
      const int64_t j0 = base + (int64_t)tid * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (j0 + i < N && (u[i] >> 21) == (uint32_t)b1) atomicAdd(&s_h[(u[i] >> 10) & 0x7ffu], 1u);
    });
    __syncthreads();
    block_find_bin_nt<kSelThreads>(s_h, kBins2, k - ab1, s_tmp, s_res, b2, ab2);
    for (int i = tid; i < kBins3; i += kSelThreads) s_h[i] = 0u;
    __syncthreads();
    const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
    sweep([&](int64_t base, const uint32_t* u) __attribute__((always_inline)) {
      const int64_t j0 = base + (int64_t)tid * PER;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (j0 + i < N && (u[i] >> 10) == pre) atomicAdd(&s_h[u[i] & 0x3ffu], 1u);
    });
    __syncthreads();
    block_find_bin_nt<kSelThreads>(s_h, kBins3, k - ab1 - ab2, s_tmp, s_res, b3, ab3);
  }
  const uint32_t tau = (((uint32_t)b1 << 11 | (uint32_t)b2) << 10) | (uint32_t)b3;
  const uint32_t r = k - ab1 - ab2 - ab3;
  int32_t* out = a.idx_out + unit * a.kk;
  // counts above / equal to tau packed in one word (each below 2^16 per step)
  uint32_t gt_run = 0, eq_run = 0;
  sweep([&](int64_t base, const uint32_t* u) __attribute__((always_inline)) {
    const int64_t j0 = base + (int64_t)tid * PER;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool in = j0 + i < N;
      gt += (in && u[i] > tau) ? 1u : 0u;
      eq += (in && u[i] == tau) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kSelThreads>((gt << 16) | eq, s_tmp, &tot);
    uint32_t g_ex = (ex >> 16) + gt_run;
    uint32_t e_ex = (ex & 0xffffu) + eq_run;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (j0 + i < N) {
        if (u[i] > tau) {
          const uint32_t pos = g_ex + min(e_ex, r);
          if (pos < k) out[pos] = (int32_t)(j0 + i);
          ++g_ex;
        } else if (u[i] == tau) {
          if (e_ex < r && g_ex + e_ex < k) out[g_ex + e_ex] = (int32_t)(j0 + i);
          ++e_ex;
        }
      }
    }
    gt_run += tot >> 16;
    eq_run += tot & 0xffffu;
  });
}

// Chunked selection, step 2 (one workgroup of 1024 threads per (b, g)): digits
// 2 and 3 of the k-th largest from the candidates (bin b1 holds it), so tau
// and r as in sel_fused_kernel; then per chunk the number of scores above tau
// (its higher-bin count plus its candidates above tau) and equal to tau, and
// their exclusive prefixes over the chunks for step 3. The candidates (the
// chunks' lists, each contiguous) are copied into LDS once, wave w taking
// chunks w, w + 16, ... with a chunk's loads issued together, and the three
// passes run there; a bin too large for LDS is read from the lists in every
// pass instead.
constexpr int kResolveCap = 16384;   // LDS candidate list of one (b, g) (64 KB)
__global__ __launch_bounds__(kSelThreads) void sel_resolve_kernel(DecodeArgs a) {
  constexpr int NW = kSelThreads / 64;
  __shared__ uint32_t s_h[kBins2];
  __shared__ uint32_t s_gt[kMaxSelChunks];
  __shared__ uint32_t s_eq[kMaxSelChunks];
  __shared__ uint32_t s_nc[kMaxSelChunks];
  __shared__ uint32_t s_off[kMaxSelChunks];
  __shared__ uint32_t s_cand[kResolveCap];
  __shared__ uint32_t s_tmp[NW];
  __shared__ int s_res[2];
  const int64_t unit = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t k = unit_k(a, unit);
  const int nch = a.n_sel_chunks;
  const uint32_t* hist1 = a.hist + unit * kHistWords;
  const uint32_t* cand = a.cand + unit * nch * (int64_t)kSelChunk;
  uint32_t* counts = a.counts + unit * nch * 2;
  for (int c = tid; c < nch; c += kSelThreads) {
    s_gt[c] = counts[2 * c];
    s_nc[c] = counts[2 * c + 1];
  }
  for (int i = tid; i < kBins2; i += kSelThreads) s_h[i] = 0u;
  int b1, b2, b3;
  uint32_t ab1, ab2, ab3;
  block_find_bin_nt<kSelThreads>(hist1, kBins1, k, s_tmp, s_res, b1, ab1);   // synchronises
  // offsets of the chunks' candidates in the LDS list
  uint32_t ncand = 0;
  for (int c0 = 0; c0 < nch; c0 += kSelThreads) {
    const int c = c0 + tid;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kSelThreads>(c < nch ? s_nc[c] : 0u, s_tmp, &tot);
    if (c < nch) s_off[c] = ncand + ex;
    ncand += tot;
  }
  __syncthreads();
  const bool staged = ncand <= (uint32_t)kResolveCap;
  if (staged) {
    for (int c = wave; c < nch; c += NW) {
      const uint32_t* cc = cand + (int64_t)c * kSelChunk;
      const uint32_t n = s_nc[c], off = s_off[c];
      for (uint32_t i0 = lane; i0 < n; i0 += 256) {
        uint32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = (i0 + 64 * q < n) ? cc[i0 + 64 * q] : 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (i0 + 64 * q < n) s_cand[off + i0 + 64 * q] = v[q];
      }
    }
    __syncthreads();
    for (uint32_t i = tid; i < ncand; i += kSelThreads) atomicAdd(&s_h[(s_cand[i] >> 10) & 0x7ffu], 1u);
  } else {
    for (int c = wave; c < nch; c += NW) {
      const uint32_t* cc = cand + (int64_t)c * kSelChunk;
      for (uint32_t i = lane; i < s_nc[c]; i += 64) atomicAdd(&s_h[(cc[i] >> 10) & 0x7ffu], 1u);
    }
  }
  __syncthreads();
  block_find_bin_nt<kSelThreads>(s_h, kBins2, k - ab1, s_tmp, s_res, b2, ab2);
  for (int i = tid; i < kBins3; i += kSelThreads) s_h[i] = 0u;
  __syncthreads();
  const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
  if (staged) {
    for (uint32_t i = tid; i < ncand; i += kSelThreads) {
      const uint32_t u = s_cand[i];
      if ((u >> 10) == pre) atomicAdd(&s_h[u & 0x3ffu], 1u);
    }
  } else {
    for (int c = wave; c < nch; c += NW) {
      const uint32_t* cc = cand + (int64_t)c * kSelChunk;
      for (uint32_t i = lane; i < s_nc[c]; i += 64) {
        const uint32_t u = cc[i];
        if ((u >> 10) == pre) atomicAdd(&s_h[u & 0x3ffu], 1u);
      }
    }
  }
  __syncthreads();
  block_find_bin_nt<kSelThreads>(s_h, kBins3, k - ab1 - ab2, s_tmp, s_res, b3, ab3);
  const uint32_t tau = (pre << 10) | (uint32_t)b3;
  const uint32_t r = k - ab1 - ab2 - ab3;
  for (int c = wave; c < nch; c += NW) {
    const uint32_t n = s_nc[c];
    const uint32_t* cc = cand + (int64_t)c * kSelChunk;
    const uint32_t* lc = s_cand + s_off[c];
    uint32_t gt = 0, eq = 0;
    for (uint32_t i = lane; i < n; i += 64) {
      const uint32_t u = staged ? lc[i] : cc[i];
      gt += u > tau ? 1u : 0u;
      eq += u == tau ? 1u : 0u;
    }
    gt = wave_sum_u32(gt);
    eq = wave_sum_u32(eq);
    if (lane == 0) {
      s_gt[c] += gt;
      s_eq[c] = eq;
    }
  }
  __syncthreads();
  // exclusive prefixes over the chunks, kSelThreads chunks at a time
  uint32_t gt_carry = 0, eq_carry = 0;
  for (int c0 = 0; c0 < nch; c0 += kSelThreads) {
    const int c = c0 + tid;
    const uint32_t g = c < nch ? s_gt[c] : 0u, e = c < nch ? s_eq[c] : 0u;
    uint32_t gtot, etot;
    const uint32_t gex = block_excl_scan<kSelThreads>(g, s_tmp, &gtot);
    const uint32_t eex = block_excl_scan<kSelThreads>(e, s_tmp, &etot);
    if (c < nch) {
      counts[2 * c] = gt_carry + gex;
      counts[2 * c + 1] = eq_carry + eex;
    }
    gt_carry += gtot;
    eq_carry += etot;
  }
  if (tid == 0) {
    a.selstate[unit * 4 + 0] = tau;
    a.selstate[unit * 4 + 1] = r;
  }
}

// ------------------------------------------------------------------ dec_attn

// One workgroup = one split of one (b, g): rows [split*split_rows, ...) of the
// index set (DENSE: of the whole cache, row i being key i). Wave w takes
// 16-row blocks w, w+4, ...; per block: Q.K^T on a 16x16 MFMA tile (or the
// anchor's stored logits), online softmax with wave-uniform running max per
// head, P.V on the VALU with 16 lanes per V row.
template <typename T, int D, int G, bool FROM_LOGITS, bool DENSE = false>
__global__ __launch_bounds__(256) void dec_attn_kernel(DecodeArgs a) {
  using QK = QKMfma<T, D>;
  constexpr int EPL = D / 16;
  __shared__ int32_t s_idx[kMaxSplitRows];
  __shared__ float s_p[4][16 * G];
  __shared__ float s_o[4][G * D];
  __shared__ float s_m[4][G], s_l[4][G];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int64_t row0 = (int64_t)split * a.split_rows;
  const int nrows = (int)min((int64_t)a.split_rows, set_rows(a, b) - row0);
  // Index values and the head map are trusted inputs; clamping keeps every
  // access inside the cache even if they are not.
  if (DENSE) {
    for (int i = tid; i < nrows; i += 256) s_idx[i] = (int32_t)(row0 + i);
  } else {
    int ga = a.head_map ? a.head_map[g] : g;
    ga = ((unsigned)ga < (unsigned)a.Hkv_a) ? ga : 0;
    const int32_t* idx = a.idx + ((int64_t)b * a.Hkv_a + ga) * a.kk + row0;
    for (int i = tid; i < nrows; i += 256) {
      const int32_t j = idx[i];
      s_idx[i] = ((uint32_t)j < (uint32_t)a.N) ? j : 0;
    }
  }
  __syncthreads();

  const int64_t unit = (int64_t)b * a.Hkv + g;
  const T* kb = (const T*)a.k + b * a.kv_bstride + kv_head(a, g) * a.kv_hstride;
  const T* vb = (const T*)a.v + b * a.kv_bstride + kv_head(a, g) * a.kv_hstride;
  const float* lg = FROM_LOGITS ? a.logits + unit * a.N * G : nullptr;

  typename QK::QFrag qf;
  if (!FROM_LOGITS)
    QK::load_q(qf, (const T*)a.q + b * a.q_bstride + (int64_t)(g * G + min(c16, G - 1)) * a.q_hstride, c16 < G, q4);

  float o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  float ml[4], ls[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { ml[r] = kNegInf; ls[r] = 0.f; }

  struct Blk {
    QK kq;
    f32x4 lgt;
    RowFrag<T, EPL> vf[4];
  };
  auto load_blk = [&](int blk, Blk& B_) {
    const int r0 = blk * 16;
    const int jr = r0 + c16;
    const int jk = s_idx[jr < nrows ? jr : 0];
    if (FROM_LOGITS) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        B_.lgt[r] = (4 * q4 + r < G) ? lg[(int64_t)jk * G + 4 * q4 + r] : 0.f;
    } else {
      B_.kq.load_k(kb + (int64_t)jk * D, q4);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jr2 = r0 + 4 * i + q4;
      const int jv = s_idx[jr2 < nrows ? jr2 : 0];
      B_.vf[i].load(vb + (int64_t)jv * D + c16 * EPL);
    }
  };

  float* sp = s_p[wave];
  const int nblk = (nrows + 15) >> 4;
  Blk cur;
  if (wave < nblk) load_blk(wave, cur);
  for (int blk = wave; blk < nblk; blk += 4) {
    Blk nxt;
    if (blk + 4 < nblk) load_blk(blk + 4, nxt);
    const bool kval = blk * 16 + c16 < nrows;
    f32x4 s;
    if (FROM_LOGITS) s = cur.lgt;
    else s = cur.kq.run(qf) * a.scale_log2;
    float t[4], p[4], al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      t[r] = kval ? s[r] : kNegInf;
      float bm = row16_max(t[r]);
      float mn = fmaxf(ml[r], bm);
      al[r] = (mn == ml[r]) ? 1.f : exp2_fast(ml[r] - mn);
      p[r] = (t[r] == kNegInf) ? 0.f : exp2_fast(t[r] - mn);
      ls[r] = ls[r] * al[r] + p[r];
      ml[r] = mn;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = readlane_f(al[h & 3], 16 * (h >> 2));
      if (ah != 1.f) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] *= ah;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * q4 + r < G) sp[c16 * G + 4 * q4 + r] = p[r];
    wave_lds_fence();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + q4;
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = sp[row * G + h];
      float vv[EPL];
      cur.vf[i].widen(vv);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] += pv[h] * vv[e];
    }
    wave_lds_fence();
    cur = nxt;
  }

  // reduce over the four lane rows (each saw different keys, same running max)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      o[h][e] += __shfl_xor(o[h][e], 16);
      o[h][e] += __shfl_xor(o[h][e], 32);
    }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float lsum = row16_sum(ls[h & 3]);
    float M = readlane_f(ml[h & 3], 16 * (h >> 2));
    float L = readlane_f(lsum, 16 * (h >> 2));
    if (lane == 0) { s_m[wave][h] = M; s_l[wave][h] = L; }
  }
  if (q4 == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wave][h * D + c16 * EPL + e] = o[h][e];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int h = x / D, d = x % D;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += (s_m[w][h] == kNegInf) ? 0.f : s_o[w][x] * exp2_fast(s_m[w][h] - M);
    a.part_o[(((int64_t)b * a.Hq + g * G + h) * a.nsplit + split) * D + d] = acc;
  }
  if (tid < G) {
    const int h = tid;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      L += (s_m[w][h] == kNegInf) ? 0.f : s_l[w][h] * exp2_fast(s_m[w][h] - M);
    float* ml_out = a.part_ml + (((int64_t)b * a.Hq + g * G + h) * a.nsplit + split) * 2;
    ml_out[0] = M;
    ml_out[1] = L;
  }
}

// Transposing LDS read (ds_read_b64_tr_b16) used by the gather's P.V operand.
typedef short dec_i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dec_i16x4 dec_lds_i16x4;
__device__ __forceinline__ u32x2 dec_lds_read_tr16(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((dec_lds_i16x4*)(p)));
}

// Pipelined 16-bit gather attention. One workgroup = one split of one (b, g);
// wave w takes 16-row blocks w, w+4, ...; per block: Q.K^T on a 16x16x32 MFMA
// tile (or the anchor's stored logits), an online softmax with a running max
// per head shared by the 16 lanes of each lane row, P (16-bit) and the
// gathered V rows staged in the wave's own LDS slice, and O += P.V on 16x16x16
// MFMA with V through the transposing LDS load. K and V rows are both loaded
// whole (16 lanes per 256-byte row) and K re-laid out into the MFMA operand
// through LDS, as in the scoring pass. Each wave keeps the K and V rows of
// its next NBUF blocks in flight in NBUF register sets, and each lane loads
// the index of its own row straight from global memory one step before the
// rows it names (V row indices are then shuffled from the lane that owns the
// row). Vector memory counters retire in issue order, so the indices of a
// block are issued before the rows of the blocks ahead of it; no load sits
// behind a divergent branch in the steady-state loop.
// DENSE: the split covers keys [row0, row0 + nrows) of the cache and a row's
// key is its position (no index loads); otherwise the same kernel.
// PG: a paged cache; the index sets hold physical rows (translated by
// dec_page_rows), addressed from k + g * page_hstride.
template <int D, int G, bool FROM_LOGITS, bool DENSE = false, typename E = __bf16, bool PG = false, bool STREAM = true>
__global__ __launch_bounds__(256, 2) void dec_gather_kernel(DecodeArgs a) {
  using QK = QKMfma<E, D>;
  constexpr int NT = D / 16;            // output tiles of 16 dims
  constexpr int VROW = 2 * D + 32;      // bytes per staged V row
  constexpr int VP = D / 8;             // 16-byte parts per V row
  constexpr int NVL = 16 * VP / 64;     // V 16-byte loads per lane per block
  // blocks in flight per wave (three measured 2.5 % faster than two at 128K
  // in both modes; four spill in reuse mode and are slower in logit mode)
  constexpr int NBUF = 3;
  __shared__ __align__(16) char s_v[4][16 * VROW];
  // K rows of the wave's block (16-byte chunks XOR-swizzled by row), re-laid
  // out from whole-row loads into the MFMA operand
  __shared__ __align__(16) char s_k[FROM_LOGITS ? 1 : 4][FROM_LOGITS ? 16 : 16 * 2 * D];
  __shared__ __align__(16) uint16_t s_p[4][16 * 16];   // [head][key] bf16; heads >= G stay 0
  __shared__ float s_o[4][G * D];
  __shared__ float s_m[4][G], s_l[4][G];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int64_t row0 = (int64_t)split * a.split_rows;
  const int nrows = (int)min((int64_t)a.split_rows, set_rows(a, b) - row0);
  const int nblk = (nrows + 15) >> 4;
  const int nb = wave < nblk ? (nblk - wave + 3) >> 2 : 0;   // blocks wave, wave + 4, ...
  int ga = (!DENSE && a.head_map) ? a.head_map[g] : g;
  ga = ((unsigned)ga < (unsigned)a.Hkv_a) ? ga : 0;
  const int32_t* idx = DENSE ? nullptr : a.idx + ((int64_t)b * a.Hkv_a + ga) * a.kk + row0;

  const int64_t unit = (int64_t)b * a.Hkv + g;
  const E* kb = PG ? (const E*)a.k + kv_head(a, g) * a.page_hstride
                  : (const E*)a.k + b * a.kv_bstride + kv_head(a, g) * a.kv_hstride;
  const E* vb = PG ? (const E*)a.v + kv_head(a, g) * a.page_hstride
                  : (const E*)a.v + b * a.kv_bstride + kv_head(a, g) * a.kv_hstride;
  const uint32_t nkeys = PG ? (uint32_t)a.pool_rows : (uint32_t)a.N;   // rows an index may name
  const float* lg = FROM_LOGITS ? a.logits + unit * a.N * G : nullptr;
  typename QK::QFrag qf;
  if (!FROM_LOGITS)
    QK::load_q(qf, (const E*)a.q + b * a.q_bstride + (int64_t)(g * G + min(c16, G - 1)) * a.q_hstride, c16 < G, q4);
  char* sv = s_v[wave];
  uint16_t* sp = s_p[wave];
  reinterpret_cast<uint32_t*>(sp)[lane] = 0u;
  reinterpret_cast<uint32_t*>(sp)[lane + 64] = 0u;

  f32x4 o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ml[4], ls[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) { ml[r] = kNegInf; ls[r] = 0.f; }

  // raw index of this lane's row (c16) in the wave's i-th block; rows past
  // the split re-read its last index and are masked in the softmax
  auto load_idx = [&](int i) -> int {
    const int blk = min(wave + 4 * i, nblk - 1);
    const int r = min(blk * 16 + c16, nrows - 1);
    if constexpr (DENSE) return (int)row0 + r;
    else return idx[r];
  };
  struct Blk {
    u32x4 k[FROM_LOGITS ? 1 : NVL];   // whole K rows, in the layout of v
    f32x4 lgt;
    u32x4 v[NVL];
  };
  // Index values are trusted inputs; clamping keeps every access inside the cache.
  // STREAM: K and V rows are loaded non-temporally. Each is read once per call,
  // and keeping them out of the caches made this kernel 9 % faster on the
  // anchor-selected sets, 34 % on uniformly random ones and 11 % in dense
  // mode (128K, batch 4). With a head map per query head (kvdiv > 1) the G
  // query heads of a KV head gather overlapping rows, which then come from
  // the caches: plain loads there.
  auto load_blk = [&](int jraw, Blk& B_) {
    const int jk = ((unsigned)jraw < nkeys) ? jraw : 0;
    if (FROM_LOGITS) {
      if constexpr (G % 4 == 0) {
        // heads 4 q4 .. 4 q4 + 3 of the key in one 16-byte load
        B_.lgt = (4 * q4 < G) ? *reinterpret_cast<const f32x4*>(lg + (int64_t)jk * G + 4 * q4) : f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) B_.lgt[r] = (4 * q4 + r < G) ? lg[(int64_t)jk * G + 4 * q4 + r] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < NVL; ++i) {
      const int x = lane + 64 * i;
      const int jv = __shfl(jk, x / VP);   // lane x / VP (< 16) owns row x / VP
      if constexpr (!FROM_LOGITS)
        B_.k[i] = STREAM ? ldg16_nt(kb + (int64_t)jv * D + (x % VP) * 8) : ldg16(kb + (int64_t)jv * D + (x % VP) * 8);
      B_.v[i] = STREAM ? ldg16_nt(vb + (int64_t)jv * D + (x % VP) * 8) : ldg16(vb + (int64_t)jv * D + (x % VP) * 8);
    }
  };
  // Whole K rows -> the Q.K^T operand (chunk 4 c + q4 of row c16 for
  // instruction c) through the wave's LDS slot; a wave's LDS accesses execute
  // in order, so one slot serves every block.
  auto k_operand = [&](const Blk& B_) __attribute__((always_inline)) -> QK {
    QK kq;
    if constexpr (!FROM_LOGITS) {
      char* sk = s_k[wave];
#pragma unroll
      for (int i = 0; i < NVL; ++i) {
        const int x = lane + 64 * i, row = x / VP, ch = x % VP;
        *reinterpret_cast<u32x4*>(sk + row * 2 * D + 16 * (ch ^ (row & (VP - 1)))) = B_.k[i];
      }
      wave_lds_fence();
#pragma unroll
      for (int c = 0; c < QK::NI; ++c)
        kq.kf[c] = *reinterpret_cast<const u32x4*>(sk + c16 * 2 * D + 16 * ((4 * c + q4) ^ (c16 & (VP - 1))));
    }
    return kq;
  };
  // transposing-read source address of this lane: key row 4*(lane/16) + (lane%16)/4,
  // dims 4*(lane%4) of each 16-dim output tile
  const char* tr_base = sv + (4 * q4 + (c16 >> 2)) * VROW + 4 * (lane & 3) * 2;

  auto process = [&](int i, const Blk& B_) {
    const int blk = wave + 4 * i;
    const f32x4 s = FROM_LOGITS ? B_.lgt : k_operand(B_).run(qf) * a.scale_log2;
    const bool kval = blk * 16 + c16 < nrows;
    float al[4];
    bool grew = false;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float t = kval ? s[r] : kNegInf;
      const float bm = row16_max(t);
      const float mn = fmaxf(ml[r], bm);
      al[r] = (mn == ml[r]) ? 1.f : exp2_fast(ml[r] - mn);
      grew |= al[r] != 1.f;
      const float p = exp2_fast(t - mn);   // -inf -> 0
      ls[r] = ls[r] * al[r] + p;
      ml[r] = mn;
      if (4 * q4 + r < G) sp[(4 * q4 + r) * 16 + c16] = Ew<E>::bits(p);
    }
    if (__any(grew)) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[n][r] *= al[r];
    }
#pragma unroll
    for (int v = 0; v < NVL; ++v) {
      const int x = lane + 64 * v;
      *reinterpret_cast<u32x4*>(sv + (x / VP) * VROW + (x % VP) * 16) = B_.v[v];
    }
    wave_lds_fence();
    const u32x2 pa = *reinterpret_cast<const u32x2*>(sp + c16 * 16 + 4 * q4);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const u32x2 vbf = dec_lds_read_tr16(tr_base + 32 * n);
      o[n] = Ew<E>::mfma16k16(pa, vbf, o[n]);
    }
    wave_lds_fence();
  };

  // NBUF register sets, indexed at compile time: the steady loop processes
  // NBUF blocks per step and refills each set right after its block, so up
  // to NBUF blocks are in flight while one is processed.
  Blk bf[NBUF];
  int jn[NBUF];
  int i = 0;
  if (nb >= 2 * NBUF) {
    // the issue order here matches the loop below, so the loop entry adds no wait
#pragma unroll
    for (int s = 0; s < NBUF; ++s) jn[s] = load_idx(s);
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      load_blk(jn[s], bf[s]);
      jn[s] = load_idx(s + NBUF);
    }
    // scheduling barriers keep each reload after the math that frees its
    // registers
    for (; i + 2 * NBUF - 1 < nb; i += NBUF) {
#pragma unroll
      for (int s = 0; s < NBUF; ++s) {
        process(i + s, bf[s]);
        __builtin_amdgcn_sched_barrier(0);
        load_blk(jn[s], bf[s]);
        jn[s] = load_idx(i + s + 2 * NBUF);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // blocks i .. nb - 1 (fewer than 2 NBUF): i + s in bf[s], indices of
    // i + NBUF + s in jn[s]
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      if (i + s < nb) process(i + s, bf[s]);
      if (i + NBUF + s < nb) load_blk(jn[s], bf[s]);
    }
#pragma unroll
    for (int s = 0; s < NBUF; ++s)
      if (i + NBUF + s < nb) process(i + NBUF + s, bf[s]);
  } else if (nb > 0) {
#pragma unroll
    for (int s = 0; s < NBUF; ++s)
      if (s < nb) load_blk(load_idx(s), bf[s]);
#pragma unroll
    for (int s = 0; s < NBUF; ++s) {
      if (s < nb) process(s, bf[s]);
      if (s + NBUF < nb) load_blk(load_idx(s + NBUF), bf[s]);
    }
#pragma unroll
    for (int s = 0; s < NBUF; ++s)
      if (s + NBUF < nb) process(s + NBUF, bf[s]);
  }

  // O rows: head 4*(lane/16) + r, dims 16 n + lane%16
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float lsum = row16_sum(ls[h & 3]);
    const float M = readlane_f(ml[h & 3], 16 * (h >> 2));
    const float L = readlane_f(lsum, 16 * (h >> 2));
    if (lane == 0) { s_m[wave][h] = M; s_l[wave][h] = L; }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * q4 + r;
    if (h < G) {
#pragma unroll
      for (int n = 0; n < NT; ++n) s_o[wave][h * D + 16 * n + c16] = o[n][r];
    }
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += 256) {
    const int h = x / D, d = x % D;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      acc += (s_m[w][h] == kNegInf) ? 0.f : s_o[w][x] * exp2_fast(s_m[w][h] - M);
    a.part_o[(((int64_t)b * a.Hq + g * G + h) * a.nsplit + split) * D + d] = acc;
  }
  if (tid < G) {
    const int h = tid;
    float M = fmaxf(fmaxf(s_m[0][h], s_m[1][h]), fmaxf(s_m[2][h], s_m[3][h]));
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      L += (s_m[w][h] == kNegInf) ? 0.f : s_l[w][h] * exp2_fast(s_m[w][h] - M);
    float* ml_out = a.part_ml + (((int64_t)b * a.Hq + g * G + h) * a.nsplit + split) * 2;
    ml_out[0] = M;
    ml_out[1] = L;
  }
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<__bf16>(__bf16* p, float x) {
  *reinterpret_cast<uint16_t*>(p) = f32_to_bf16_rne(x);
}
template <>
__device__ __forceinline__ void store_out<_Float16>(_Float16* p, float x) {
  *reinterpret_cast<uint16_t*>(p) = Ew<_Float16>::bits(x);
}

// Merge of the split-K partials of one (b, query head): weights
// exp2(m_s - M) staged in LDS, 256 threads = (256 / D) interleaved split
// streams per output dim.
template <typename T>
__global__ __launch_bounds__(256) void dec_combine_kernel(DecodeArgs a) {
  constexpr int WCH = 1024;
  __shared__ float s_w[WCH];
  __shared__ float s_tmp[4];
  __shared__ float s_acc[256];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t bh = (int64_t)b * a.Hq + h;
  const float* ml = a.part_ml + bh * a.nsplit * 2;
  const float* po = a.part_o + bh * a.nsplit * a.D;
  float m = kNegInf;
  for (int s = tid; s < a.nsplit; s += 256) m = fmaxf(m, ml[2 * s]);
  const float M = block_max_256(m, s_tmp);
  float l = 0.f;
  for (int s = tid; s < a.nsplit; s += 256) l += ml[2 * s + 1] * exp2_fast(ml[2 * s] - M);
  const float L = block_sum_256(l, s_tmp);
  const int D = a.D, nparts = 256 / D, d = tid % D, part = tid / D;
  float acc = 0.f;
  for (int s0 = 0; s0 < a.nsplit; s0 += WCH) {
    const int n = min(WCH, a.nsplit - s0);
    __syncthreads();
    for (int i = tid; i < n; i += 256) s_w[i] = exp2_fast(ml[2 * (s0 + i)] - M);
    __syncthreads();
#pragma unroll 4
    for (int i = part; i < n; i += nparts) acc += po[(int64_t)(s0 + i) * D + d] * s_w[i];
  }
  s_acc[tid] = acc;
  __syncthreads();
  if (part == 0) {
    float tot = 0.f;
    for (int x = 0; x < nparts; ++x) tot += s_acc[x * D + d];
    store_out<T>((T*)a.o + b * a.o_bstride + (int64_t)h * a.o_hstride + d, tot / L);
  }
}

// ------------------------------------------------------------------ launchers

#define KAS_LAUNCH(kernel, grid, block, ctx, arg) (ctx).launch(kernel, grid, block, arg)

template <typename T, int D, bool PG>
static hipError_t score_launch_pg(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  switch (a.G) {
    case 1: KAS_LAUNCH((dec_score_kernel<T, D, 1, PG>), grid, dim3(256), st, a); break;
    case 2: KAS_LAUNCH((dec_score_kernel<T, D, 2, PG>), grid, dim3(256), st, a); break;
    case 4: KAS_LAUNCH((dec_score_kernel<T, D, 4, PG>), grid, dim3(256), st, a); break;
    case 8: KAS_LAUNCH((dec_score_kernel<T, D, 8, PG>), grid, dim3(256), st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}
template <typename T, int D, bool PG>
static hipError_t score_launch_ix_pg(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  switch (a.G) {
    case 1: KAS_LAUNCH((dec_score_kernel<T, D, 1, PG, true>), grid, dim3(256), st, a); break;
    case 2: KAS_LAUNCH((dec_score_kernel<T, D, 2, PG, true>), grid, dim3(256), st, a); break;
    case 4: KAS_LAUNCH((dec_score_kernel<T, D, 4, PG, true>), grid, dim3(256), st, a); break;
    case 8: KAS_LAUNCH((dec_score_kernel<T, D, 8, PG, true>), grid, dim3(256), st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}
template <typename T, int D>
static hipError_t score_launch_ix(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  if (sizeof(T) == 2 && a.block_table) return score_launch_ix_pg<T, D, true>(a, grid, st);
  return score_launch_ix_pg<T, D, false>(a, grid, st);
}

hipError_t launch_decode_score_pool_rows(const DecodeArgs& a, int dtype, LaunchCtx& ctx) {
  dim3 grid(a.n_score_chunks, a.Hkv, a.B);
  ctx.begin(K_DEC_SCORE);
  hipError_t e;
  if (dtype == 1) e = a.D == 128 ? score_launch_ix<__bf16, 128>(a, grid, ctx) : score_launch_ix<__bf16, 64>(a, grid, ctx);
  else if (dtype == 2) e = a.D == 128 ? score_launch_ix<_Float16, 128>(a, grid, ctx) : score_launch_ix<_Float16, 64>(a, grid, ctx);
  else e = a.D == 128 ? score_launch_ix<float, 128>(a, grid, ctx) : score_launch_ix<float, 64>(a, grid, ctx);
  if (e != hipSuccess) return e;
  return ctx.end(K_DEC_SCORE);
}

template <typename T, int D>
static hipError_t score_launch(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  // paged caches hold 16-bit elements only (checked on the host)
  if (sizeof(T) == 2 && a.block_table) return score_launch_pg<T, D, true>(a, grid, st);
  return score_launch_pg<T, D, false>(a, grid, st);
}

hipError_t launch_decode_score(const DecodeArgs& a, int dtype, LaunchCtx& ctx) {
  dim3 grid(a.n_score_chunks, a.Hkv, a.B);
  ctx.begin(K_DEC_SCORE);
  hipError_t e;
  if (dtype == 1) e = (a.D == 128) ? score_launch<__bf16, 128>(a, grid, ctx)
                                   : score_launch<__bf16, 64>(a, grid, ctx);
  else if (dtype == 2) e = (a.D == 128) ? score_launch<_Float16, 128>(a, grid, ctx)
                                        : score_launch<_Float16, 64>(a, grid, ctx);
  else e = (a.D == 128) ? score_launch<float, 128>(a, grid, ctx)
                        : score_launch<float, 64>(a, grid, ctx);
  if (e != hipSuccess) return e;
  return ctx.end(K_DEC_SCORE);
}

template <int OP, bool ALL>
static hipError_t pool_launch(const DecodeArgs& a, dim3 grid, LaunchCtx& ctx) {
  switch (a.G) {
    case 1: KAS_LAUNCH((dec_pool_kernel<1, OP, ALL>), grid, dim3(256), ctx, a); break;
    case 2: KAS_LAUNCH((dec_pool_kernel<2, OP, ALL>), grid, dim3(256), ctx, a); break;
    case 4: KAS_LAUNCH((dec_pool_kernel<4, OP, ALL>), grid, dim3(256), ctx, a); break;
    case 8: KAS_LAUNCH((dec_pool_kernel<8, OP, ALL>), grid, dim3(256), ctx, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

hipError_t launch_decode_pool(const DecodeArgs& a, LaunchCtx& ctx) {
  dim3 grid(a.n_sel_chunks, a.pool_all ? 1 : a.Hkv, a.B);
  ctx.begin(K_DEC_POOL);
  hipError_t e;
  if (a.pool_all) e = a.pool_op ? pool_launch<1, true>(a, grid, ctx) : pool_launch<0, true>(a, grid, ctx);
  else e = a.pool_op ? pool_launch<1, false>(a, grid, ctx) : pool_launch<0, false>(a, grid, ctx);
  if (e != hipSuccess) return e;
  return ctx.end(K_DEC_POOL);
}

hipError_t launch_decode_select(const DecodeArgs& a, LaunchCtx& ctx) {
  // the one-workgroup-per-set kernel: when selected by the tuning option, by
  // default for sets of at most two chunks (one launch instead of three:
  // 58 against 63 us for a 2K anchor layer, even at 32K, 26 us slower at
  // 128K), and when there are more chunks than the chunked path resolves in LDS
  const int64_t one = option_value(KAS_OPT_DECODE_SELECT_ONE_PASS);
  if (one == 1 || (one == -1 && a.n_sel_chunks <= 2) || a.n_sel_chunks > kMaxSelChunks) {
    ctx.begin(K_SEL_FUSED);
    KAS_LAUNCH(sel_fused_kernel, dim3((unsigned)a.sel_units), dim3(kSelThreads), ctx, a);
    return ctx.end(K_SEL_FUSED);
  }
  dim3 grid(a.n_sel_chunks, (unsigned)a.sel_units);
  hipError_t e;
  ctx.begin(K_SEL_CAND);
  KAS_LAUNCH(sel_cand_kernel, grid, dim3(256), ctx, a);
  if ((e = ctx.end(K_SEL_CAND)) != hipSuccess) return e;
  ctx.begin(K_SEL_RESOLVE);
  KAS_LAUNCH(sel_resolve_kernel, dim3((unsigned)a.sel_units), dim3(kSelThreads), ctx, a);
  if ((e = ctx.end(K_SEL_RESOLVE)) != hipSuccess) return e;
  ctx.begin(K_SEL_COMPACT);
  KAS_LAUNCH(sel_compact_kernel, grid, dim3(256), ctx, a);
  return ctx.end(K_SEL_COMPACT);
}

template <typename T, int D, bool FL, bool DENSE = false>
static hipError_t attn_launch(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  switch (a.G) {
    case 1: KAS_LAUNCH((dec_attn_kernel<T, D, 1, FL, DENSE>), grid, dim3(256), st, a); break;
    case 2: KAS_LAUNCH((dec_attn_kernel<T, D, 2, FL, DENSE>), grid, dim3(256), st, a); break;
    case 4: KAS_LAUNCH((dec_attn_kernel<T, D, 4, FL, DENSE>), grid, dim3(256), st, a); break;
    case 8: KAS_LAUNCH((dec_attn_kernel<T, D, 8, FL, DENSE>), grid, dim3(256), st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

template <typename T, bool FL, bool DENSE = false>
static hipError_t attn_by_d(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  return a.D == 128 ? attn_launch<T, 128, FL, DENSE>(a, grid, st) : attn_launch<T, 64, FL, DENSE>(a, grid, st);
}

template <int D, bool FL, bool DENSE = false, typename E = __bf16, bool PG = false>
static hipError_t gather_launch(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  switch (a.G) {
    case 1:   // a head map per query head runs its heads as groups of one (kvdiv > 1)
      if (a.kvdiv > 1) KAS_LAUNCH((dec_gather_kernel<D, 1, FL, DENSE, E, PG, false>), grid, dim3(256), st, a);
      else KAS_LAUNCH((dec_gather_kernel<D, 1, FL, DENSE, E, PG>), grid, dim3(256), st, a);
      break;
    case 2: KAS_LAUNCH((dec_gather_kernel<D, 2, FL, DENSE, E, PG>), grid, dim3(256), st, a); break;
    case 4: KAS_LAUNCH((dec_gather_kernel<D, 4, FL, DENSE, E, PG>), grid, dim3(256), st, a); break;
    case 8: KAS_LAUNCH((dec_gather_kernel<D, 8, FL, DENSE, E, PG>), grid, dim3(256), st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}
template <bool FL>
static hipError_t attn_bf16_by_d(const DecodeArgs& a, dim3 grid, LaunchCtx& st) {
  return a.D == 128 ? gather_launch<128, FL>(a, grid, st) : gather_launch<64, FL>(a, grid, st);
}

// merge of the split partials into o
static hipError_t launch_combine(const DecodeArgs& a, int dtype, LaunchCtx& ctx) {
  ctx.begin(K_DEC_COMBINE);
  dim3 cgrid(a.Hq, a.B);
  if (dtype == 1) KAS_LAUNCH((dec_combine_kernel<__bf16>), cgrid, dim3(256), ctx, a);
  else if (dtype == 2) KAS_LAUNCH((dec_combine_kernel<_Float16>), cgrid, dim3(256), ctx, a);
  else KAS_LAUNCH((dec_combine_kernel<float>), cgrid, dim3(256), ctx, a);
  return ctx.end(K_DEC_COMBINE);
}

// Paged caches: the gather over translated physical rows (from_logits is
// not used: the rows' own K is read again).
static hipError_t gather_paged(const DecodeArgs& a, int dtype, dim3 grid, LaunchCtx& ctx) {
  if (dtype == 1)
    return a.D == 128 ? gather_launch<128, false, false, __bf16, true>(a, grid, ctx)
                      : gather_launch<64, false, false, __bf16, true>(a, grid, ctx);
  if (dtype == 2)
    return a.D == 128 ? gather_launch<128, false, false, _Float16, true>(a, grid, ctx)
                      : gather_launch<64, false, false, _Float16, true>(a, grid, ctx);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_attn(const DecodeArgs& a, int dtype, bool from_logits, LaunchCtx& ctx) {
  dim3 grid(a.nsplit, a.Hkv, a.B);
  hipError_t e;
  const int kid = from_logits ? K_DEC_ATTN_ANCHOR : K_DEC_ATTN;
  ctx.begin(kid);
  if (a.block_table) e = gather_paged(a, dtype, grid, ctx);
  else if (dtype == 1) e = from_logits ? attn_bf16_by_d<true>(a, grid, ctx)
                                  : attn_bf16_by_d<false>(a, grid, ctx);
  else if (dtype == 2)
    e = from_logits ? (a.D == 128 ? gather_launch<128, true, false, _Float16>(a, grid, ctx)
                                  : gather_launch<64, true, false, _Float16>(a, grid, ctx))
                    : (a.D == 128 ? gather_launch<128, false, false, _Float16>(a, grid, ctx)
                                  : gather_launch<64, false, false, _Float16>(a, grid, ctx));
  else e = from_logits ? attn_by_d<float, true>(a, grid, ctx)
                       : attn_by_d<float, false>(a, grid, ctx);
  if (e != hipSuccess) return e;
  if ((e = ctx.end(kid)) != hipSuccess) return e;
  return launch_combine(a, dtype, ctx);
}

hipError_t launch_decode_dense(const DecodeArgs& a, int dtype, LaunchCtx& ctx) {
  dim3 grid(a.nsplit, a.Hkv, a.B);
  hipError_t e;
  ctx.begin(K_DEC_DENSE);
  if (a.block_table)   // the sets are the translated rows of keys 0 .. seq_len - 1
    e = gather_paged(a, dtype, grid, ctx);
  else if (dtype == 1)
    e = a.D == 128 ? gather_launch<128, false, true>(a, grid, ctx) : gather_launch<64, false, true>(a, grid, ctx);
  else if (dtype == 2)
    e = a.D == 128 ? gather_launch<128, false, true, _Float16>(a, grid, ctx)
                   : gather_launch<64, false, true, _Float16>(a, grid, ctx);
  else
    e = attn_by_d<float, false, true>(a, grid, ctx);
  if (e != hipSuccess) return e;
  if ((e = ctx.end(K_DEC_DENSE)) != hipSuccess) return e;
  return launch_combine(a, dtype, ctx);
}

// ------------------------------------------------------------------ paged caches

// Physical row of every key in this call's sets: key j of sequence b sits in
// page block_table[b][j >> page_shift] at row j & (P - 1); rows are counted
// in D elements from k + g * page_hstride, so a page starts at row
// page * page_stride / D. One workgroup per (chunk of the set, set, b); set s
// reads source set head_map[s] (or s, clamped to the source's sets), or the
// keys themselves when there is no source.
__global__ __launch_bounds__(256) void dec_page_rows_kernel(DecodeArgs a) {
  const int s = blockIdx.y, b = blockIdx.z;
  const int64_t rows = set_rows(a, b), n = seq_n(a, b);
  int ga = (a.page_src && a.head_map) ? a.head_map[s] : s;
  ga = ((unsigned)ga < (unsigned)a.page_src_sets) ? ga : 0;
  const int32_t* in = a.page_src ? a.page_src + ((int64_t)b * a.page_src_sets + ga) * a.kk : nullptr;
  uint32_t* out = a.prow + ((int64_t)b * gridDim.y + s) * a.kk;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int64_t page_rows = a.page_stride / a.D;
  const int64_t mask = (int64_t(1) << a.page_shift) - 1;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows; i += (int64_t)gridDim.x * 256) {
    int64_t j = in ? (int64_t)in[i] : i;
    j = ((uint64_t)j < (uint64_t)n) ? j : 0;            // trusted input, kept in the sequence
    out[i] = (uint32_t)(page_id(a, bt[j >> a.page_shift]) * page_rows + (j & mask));
  }
}

// Refined layer: the selected positions in each (b, g)'s pool, in ascending
// order, mapped to the pool's keys (also ascending, so the set stays sorted).
__global__ __launch_bounds__(256) void dec_pool_keys_kernel(DecodeArgs a) {
  const int g = blockIdx.y, b = blockIdx.z;
  int ga = a.head_map ? a.head_map[g] : g;
  ga = ((unsigned)ga < (unsigned)a.Hkv_a) ? ga : 0;
  const int32_t* pool = a.idx + ((int64_t)b * a.Hkv_a + ga) * a.N;
  const int32_t* pos = a.pos + ((int64_t)b * a.Hkv + g) * a.kk;
  int32_t* out = a.idx_out + ((int64_t)b * a.Hkv + g) * a.kk;
  const int64_t rows = set_rows(a, b);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows; i += (int64_t)gridDim.x * 256) {
    const int32_t p = pos[i];
    out[i] = pool[((uint32_t)p < (uint64_t)a.N) ? p : 0];
  }
}

hipError_t launch_pool_positions_to_keys(const DecodeArgs& a, LaunchCtx& ctx) {
  ctx.begin(K_DEC_REFINE_MAP);
  const int64_t chunks = (a.kk + 255) / 256;
  KAS_LAUNCH(dec_pool_keys_kernel, dim3((unsigned)(chunks < 16 ? chunks : 16), a.Hkv, a.B), dim3(256), ctx, a);
  return ctx.end(K_DEC_REFINE_MAP);
}

struct RefineLens {
  const int32_t* seq_lens;
  const int32_t* pool_lens;
  int B, pct;
  int64_t N, pool_size;
  int32_t* pool_out;
  int32_t* kappa_out;
};

__global__ __launch_bounds__(256) void dec_refine_lens_kernel(RefineLens r) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= r.B) return;
  int64_t L = r.seq_lens ? (int64_t)r.seq_lens[b] : r.N;
  L = L < 1 ? 1 : (L > r.N ? r.N : L);
  const int64_t cap = r.pool_size < L ? r.pool_size : L;
  int64_t n = r.pool_lens ? (int64_t)r.pool_lens[b] : r.pool_size;
  n = n < 1 ? 1 : (n > cap ? cap : n);
  const int64_t k = decode_k_of(L, r.pct);
  r.pool_out[b] = (int32_t)n;
  r.kappa_out[b] = (int32_t)(k < n ? k : n);
}

hipError_t launch_refine_lens(const int32_t* seq_lens, const int32_t* pool_lens, int B, int64_t N,
                              int64_t pool_size, int pct, int32_t* pool_out, int32_t* kappa_out, LaunchCtx& ctx) {
  ctx.begin(K_DEC_REFINE_LENS);
  const RefineLens r{seq_lens, pool_lens, B, pct, N, pool_size, pool_out, kappa_out};
  KAS_LAUNCH(dec_refine_lens_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), ctx, r);
  return ctx.end(K_DEC_REFINE_LENS);
}

hipError_t launch_page_rows(const DecodeArgs& a, int nsets, LaunchCtx& ctx) {
  ctx.begin(K_DEC_PAGE_ROWS);
  const int64_t chunks = (a.kk + 255) / 256;
  dim3 grid((unsigned)(chunks < 64 ? chunks : 64), nsets, a.B);
  KAS_LAUNCH(dec_page_rows_kernel, grid, dim3(256), ctx, a);
  return ctx.end(K_DEC_PAGE_ROWS);
}

}  // namespace kas
