// Prefill-phase kernels for gfx950: query tiles of 32 rows, 16-bit inputs
// (bf16 or fp16, the element type E of the matrix kernels), 32x32x16 MFMA
// tiles of that type, fp32 softmax.
//
//  pre_offsets  CSR offsets of the per-tile index sets.
//  pre_stats    pass 1 of the anchor: for every query row its base-2
//               log-sum-exp over the causal row (S^T = K.Q^T tiles, so each
//               lane owns one query row and 16 keys of every 32-key block).
//  pre_pool     pass 2 of the anchor: S = Q.K^T tiles over the keys before
//               the tile, post-softmax probabilities exp2(s - lse), summed
//               over the tile's 32 rows and the group's G heads (Kascade
//               README "Abstract": tile-level, head-aware post-softmax
//               pooling). Each lane owns one key of the block.
//  pre_select   exact Top-k_t of each tile's pooled row (radix select over
//               the fp32 bit pattern, ties to the lower index; the first
//               digit's bin comes from pre_pool), written as ascending CSR
//               indices.
//  pre_attn     anchor output and reuse layers: one workgroup per (tile, KV
//               head), gathered K rows and transposed V rows in LDS, S^T and
//               P.V on MFMA, online softmax over the tile's index set plus
//               its causal diagonal block.
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "kas_block.hpp"
#include "kas_prefill.hpp"

namespace kas {

// Pooled-score buffer cap: one pooling launch covers a 128K prompt with 8 KV
// heads (8.6 GB), which beats chunked launches (fewer launch tails); the
// buffer is only as large as the prompt needs.
constexpr int kPoolBudgetMBDefault = 16384;

// Tiles of sequence b: all T, or its own length's (a trusted input, clamped
// to [1 tile, N] and taken in whole tiles). Tiles past it are not computed:
// causality keeps every earlier tile's work inside the sequence.
__device__ __forceinline__ int tiles_in(const int32_t* lens, int b, int64_t N, int T) {
  if (!lens) return T;
  int64_t n = lens[b];
  n = n < kTile ? kTile : (n > N ? N : n);
  return (int)(n / kTile);
}
__device__ __forceinline__ int tiles_of(const PrefillArgs& a, int b) { return tiles_in(a.seq_lens, b, a.N, a.T); }

// Row (query or key) of the 32x32 MFMA output held by lane half hh in reg r.
__device__ __forceinline__ int mrow(int r, int hh) { return 8 * (r >> 2) + 4 * hh + (r & 3); }

__device__ __forceinline__ int64_t dev_topk_count(int64_t n, int pct) {
  if (n <= 0) return 0;
  int64_t k = ((int64_t)pct * n + 50) / 100;
  return k > n ? n : k;
}

// Pooled-row slot of (b, g, t) inside a launch covering tiles [ta, tb).
__device__ __forceinline__ int64_t pool_slot(const PrefillArgs& a, int b, int g, int t) {
  const int64_t units = (int64_t)a.B * a.Hkv;
  const int64_t before = (int64_t)t * (t - 1) / 2 - (int64_t)a.t_begin * (a.t_begin - 1) / 2;
  return (before * units + ((int64_t)b * a.Hkv + g) * t) * kTile;
}

// ------------------------------------------------------------------ offsets

__global__ __launch_bounds__(256) void pre_offsets_kernel(PrefillArgs a) {
  __shared__ uint32_t s_tmp[4];
  int64_t carry = 0;
  for (int base = 0; base < a.T; base += 256) {
    const int t = base + threadIdx.x;
    const uint32_t kt = t < a.T ? (uint32_t)dev_topk_count((int64_t)t * kTile, a.pct) : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan_256(kt, s_tmp, &tot);
    if (t < a.T) a.offsets[t] = (int32_t)(carry + ex);
    carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.offsets[a.T] = (int32_t)carry;
}

// ------------------------------------------------------------------ XCD-aware order

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2). Within every group of 64 consecutive workgroups, the 8 that land on
// one XCD get 8 consecutive work items (adjacent tiles share K/V rows and
// index sets). Items are otherwise processed longest first.
__device__ __forceinline__ int xcd_local_order(int j, int n) {
  const int base = j & ~63;
  if (base + 64 > n) return j;
  const int w = j & 63;
  return base + (w & 7) * 8 + (w >> 3);
}

// Work item of workgroup j in a one-dimensional grid of n items for each of
// `units` units (unit = b * hkv + g; item 0 is a unit's longest, the cost of
// an item falling with its index). Global order: the items of all units run
// longest first, in groups of 8 adjacent items of one unit, so that no unit's
// longest items start near the end of the grid. Otherwise each unit's items
// run in turn, longest first, which keeps one head's K and V rows together in
// the caches. Either way the 8 workgroups of a group of 8 consecutive items
// land on one XCD (xcd_local_order).
struct WorkItem { int i, g, b; };
constexpr int kAttnGlobalOrderTiles = 2048;   // tile attention: global order below this many tiles
__device__ __forceinline__ WorkItem work_item(int j, int n, int hkv, int units, bool global) {
  const int k = xcd_local_order(j, n * units);
  int i, u;
  if (!global) {
    u = k / n;
    i = k - u * n;
  } else {
    const int full = n >> 3;                 // complete groups of 8 per unit
    const int in_full = full * 8 * units;
    if (k < in_full) {
      const int grp = k / (8 * units), r = k - grp * 8 * units;
      i = grp * 8 + (r & 7);
      u = r >> 3;
    } else {
      const int tail = n - full * 8, r = k - in_full;
      u = r / tail;
      i = full * 8 + (r - u * tail);
    }
  }
  return {i, u % hkv, u / hkv};
}

// ------------------------------------------------------------------ K block staging

// s_waitcnt immediate (gfx9 encoding) waiting for vector memory only:
// vmcnt in bits 3:0 and 15:14, expcnt (6:4) and lgkmcnt (11:8) left at max.
__host__ __device__ constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
// the same with lgkmcnt 0 as well (LDS stores done)
__host__ __device__ constexpr int vmcnt_lgkm0_imm(int n) { return vmcnt_imm(n) & ~0x0F00; }

// Word 3 of a raw (untyped) buffer resource: 32-bit data format, which the
// buffer unit requires to be non-zero; stride 0, so num_records counts bytes.
constexpr int kBufWord3 = 0x00020000;

// 16-byte chunk swizzles of unpadded K and V rows in LDS (64 banks of 4 B).
// K rows are read row-per-lane, 16 lanes (16 rows) per 16-byte read phase; V
// rows by the transposing read (4 rows x 2 chunks per 16-lane group); the XOR
// keeps each phase on distinct banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }


// 32 consecutive K rows of one (b, g) straight into an LDS stage by DMA
// (buffer_load_dwordx4 ... lds through a buffer resource over the slice, so
// row offsets are 32-bit), unpadded with the 16-byte chunks swizzled per row
// by swz_k: LDS slot (row, s) holds global chunk s ^ swz_k(row), and a reader
// wanting chunk c of row r reads slot c ^ swz_k(r). A block is NINS 1 KB
// lines; wave w issues lines w, w + G, ... (NIW per wave, all waves equally
// many when EVEN).
template <int D, int G>
struct KDma {
  static constexpr int ROWB = 2 * D, BLKB = 32 * ROWB, PARTS = D / 8, RPI = 64 / PARTS;
  static constexpr int NINS = 32 / RPI, NIW = (NINS + G - 1) / G;
  static constexpr bool EVEN = NINS % G == 0;
  __amdgpu_buffer_rsrc_t rk;
  int w, lrow, lslot;
  __device__ __forceinline__ void init(const void* kbase, int64_t nrows) {
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, (int)(nrows * ROWB), kBufWord3);
    w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    lrow = lane / PARTS;
    lslot = lane % PARTS;
  }
  __device__ __forceinline__ void issue(int row0, char* dst) const {
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int i = w + G * j;
      if (EVEN || i < NINS) {
        const int r = RPI * i + lrow;
        const int off = (row0 + r) * ROWB + 16 * (lslot ^ swz_k<D>(r));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16,
                                                 off, 0, 0, 0);
      }
    }
  }
  // chunk c (16 bytes) of row `row` of a staged block
  __device__ __forceinline__ static const u32x4& read(const char* stage, int row, int c) {
    return *reinterpret_cast<const u32x4*>(stage + row * ROWB + 16 * (c ^ swz_k<D>(row)));
  }
};

// ------------------------------------------------------------------ pass 1: row statistics

// Online (max, sum of exp) of one lane's query row over the 16 keys it holds
// in a 32x32 S^T tile.
__device__ __forceinline__ void row_stats_update(const f32x16& acc, bool diag, int n32, int hh, float cs,
                                                 float& m, float& l) {
  float v[16];
  if (diag) {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = (mrow(r, hh) > n32) ? kNegInf : acc[r];
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = acc[r];
  }
  float bm = fmaxf(fmaxf(v[0], v[1]), v[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) bm = fmaxf(fmaxf(bm, v[r]), v[r + 1]);
  bm = fmaxf(bm, v[15]);
  const float mn = fmaxf(m, bm * cs);
  if (mn != kNegInf) {
    const float al = (mn == m) ? 1.f : exp2_fast(m - mn);
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += exp2_fast(fmaf(v[r], cs, -mn));
    l = l * al + s;
    m = mn;
  }
}

// One workgroup = two consecutive tiles (t0 = 2p, t1 = 2p+1) of one KV head;
// wave w = query head g*G + w; each staged K block feeds both tiles.
template <int D, int G, typename E = __bf16>
__global__ __launch_bounds__(64 * G, 2) void pre_stats_kernel(PrefillArgs a) {
  constexpr int KC = D / 16;
  using KD = KDma<D, G>;
  // three K stages, filled two blocks ahead (distinct arrays, so the
  // compiler tells the stage being read from the stage being filled)
  __shared__ __align__(1024) char s_k0[KD::BLKB];
  __shared__ __align__(1024) char s_k1[KD::BLKB];
  __shared__ __align__(1024) char s_k2[KD::BLKB];
  const int npairs = (a.T + 1) / 2;
  const WorkItem it = work_item(blockIdx.x, npairs, a.Hkv, a.Hkv * a.B, true);
  const int p = npairs - 1 - it.i;
  const int g = it.g, b = it.b;
  const int t0 = 2 * p, t1 = 2 * p + 1;
  const int Tb = tiles_of(a, b);
  if (t0 >= Tb) return;                           // past the sequence (whole workgroup)
  const bool has1 = t1 < Tb;
  const int tl = has1 ? t1 : t0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n32 = lane & 31, hh = lane >> 5;
  const int h = g * G + w;
  const int64_t lse_off = ((int64_t)b * a.Hq + h) * a.N;   // row statistics of this head
  u32x4 qb0[KC], qb1[KC];
  {
    const E* qh = (const E*)a.q + b * a.q_bstride + h * a.q_hstride;
    const E* q0 = qh + (int64_t)(kTile * t0 + n32) * a.q_tstride;
    const E* q1 = qh + (int64_t)(kTile * (has1 ? t1 : t0) + n32) * a.q_tstride;
#pragma unroll
    for (int c = 0; c < KC; ++c) { qb0[c] = ldg16(q0 + 16 * c + 8 * hh); qb1[c] = ldg16(q1 + 16 * c + 8 * hh); }
  }
  const E* kbase = (const E*)a.k + b * a.kv_bstride + g * a.kv_hstride;
  const float cs = a.scale_log2;
  KD kd;
  kd.init(kbase, a.N);
  // Row sums against a lazy reference: each lane keeps a base-2 offset mr
  // (the maximum of its first block) and adds exp2(x - mr) of every later
  // score; the terms stay below 2^64 unless a score exceeds mr by 64, and
  // only such a block (rare) is redone against its own maximum. Besides the
  // MFMA, a score costs one FMA, one exponential and one add, and the update
  // has no branch, so it can share a basic block with the other tile's MFMA
  // chain.
  constexpr float kBig = 0x1p64f;
  float mr0 = 0.f, l0 = 0.f, mr1 = 0.f, l1 = 0.f;
  auto chain = [&](const u32x4* ka, const u32x4* qb) __attribute__((always_inline)) {
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) acc = Ew<E>::mfma32(ka[c], qb[c], acc);   // S^T[key][query]
    return acc;
  };
  auto stage = [&](auto st_tag) __attribute__((always_inline)) -> char* {
    constexpr int ST = decltype(st_tag)::value;
    return ST == 0 ? s_k0 : (ST == 1 ? s_k1 : s_k2);
  };
  auto read_k = [&](auto st_tag, u32x4* ka) __attribute__((always_inline)) {
    const char* sk = stage(st_tag);
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = KD::read(sk, n32, 2 * c + hh);
  };
  // masked score (diagonal block: keys after the query row are excluded)
  auto val = [&](const f32x16& acc, int r, bool diag) __attribute__((always_inline)) -> float {
    return (diag && mrow(r, hh) > n32) ? kNegInf : acc[r];
  };
  auto block_max = [&](const f32x16& acc, bool diag) __attribute__((always_inline)) -> float {
    float bm = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) bm = fmaxf(bm, val(acc, r, diag));
    return bm == kNegInf ? 0.f : bm * cs;      // all masked: any finite reference
  };
  auto terms = [&](const f32x16& acc, bool diag, float mr) __attribute__((always_inline)) -> float {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += exp2_fast(fmaf(val(acc, r, diag), cs, -mr));
    return s;
  };
  // An MFMA chain with the exponential terms of an earlier, independent block
  // woven in: 16 / KC terms after each MFMA, pinned by scheduling barriers so
  // the VALU work fills the matrix unit's dependent-chain latency.
  auto chain_terms = [&](const u32x4* ka, const u32x4* qb, const f32x16& prev, bool pdiag, float mr,
                         float& s) __attribute__((always_inline)) {
    constexpr int TPM = 16 / KC;
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      // terms first: the first group covers the LDS latency of ka[0]
#pragma unroll
      for (int e = 0; e < TPM; ++e) s += exp2_fast(fmaf(val(prev, TPM * c + e, pdiag), cs, -mr));
      acc = Ew<E>::mfma32(ka[c], qb[c], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };
  auto settle = [&](const f32x16& acc, bool diag, float s, float& mr, float& l) __attribute__((always_inline)) {
    const bool over = !(s <= kBig);
    if (__builtin_expect(__any(over), 0)) {
      if (over) {
        const float mn = fmaxf(mr, block_max(acc, diag));
        l = l * exp2_fast(mr - mn) + terms(acc, diag, mn);
        mr = mn;
        return;
      }
    }
    l += s;
  };
  // Block kb is in stage kb % 3 (ST). Before its math: the DMA of block
  // kb + 2 into stage (ST + 2) % 3 (block kb - 1's, released by the last
  // barrier). After it: block kb + 1 has landed in this wave (only the lines
  // just issued may still be in flight; said with the builtin wait, which the
  // compiler's own wait placement sees), then a barrier without a fence (the
  // block's LDS reads were consumed by its MFMAs).
  // (STEADY: block kb + 2 exists, so the DMA and the partial wait need no test)
  auto begin = [&](int kb, auto st_tag, auto steady_tag) __attribute__((always_inline)) {
    using S2 = std::integral_constant<int, (decltype(st_tag)::value + 2) % 3>;
    if (decltype(steady_tag)::value || kb + 2 <= tl) kd.issue(kTile * (kb + 2), stage(S2{}));
  };
  auto end = [&](int kb, auto steady_tag) __attribute__((always_inline)) {
    if (KD::EVEN && (decltype(steady_tag)::value || kb + 2 <= tl)) __builtin_amdgcn_s_waitcnt(vmcnt_imm(KD::NIW));
    else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2 = std::integral_constant<int, 2>;
  // fn(st_tag) with the stage of block kb named at compile time
  auto on_stage = [&](int kb, auto&& fn) __attribute__((always_inline)) {
    const int st = kb % 3;
    if (st == 0) fn(St0{});
    else if (st == 1) fn(St1{});
    else fn(St2{});
  };
  kd.issue(0, s_k0);
  if (tl >= 1) kd.issue(kTile, s_k1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  u32x4 ka[KC];
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (has1) {
    f32x16 acc1 = {};
    // One key block for both tiles. Tile 1's update of the previous block
    // runs beside tile 0's MFMA chain, tile 0's update beside tile 1's chain.
    // FIRST: block 0 (references set, no previous tile-1 block); DIAG0: block
    // t0 is tile 0's diagonal.
    auto iter = [&](int kb, auto first_tag, auto diag0_tag, auto st_tag, auto steady_tag) __attribute__((always_inline)) {
      constexpr bool FIRST = decltype(first_tag)::value, DIAG0 = decltype(diag0_tag)::value;
      begin(kb, st_tag, steady_tag);
      read_k(st_tag, ka);
      float s1 = 0.f, s0 = 0.f;
      const f32x16 acc0 = FIRST ? chain(ka, qb0) : chain_terms(ka, qb0, acc1, false, mr1, s1);
      if (FIRST) mr0 = block_max(acc0, DIAG0);
      const f32x16 acc1n = chain_terms(ka, qb1, acc0, DIAG0, mr0, s0);
      // keep the sums where they are computed (not sunk into the branches below)
      asm volatile("" : "+v"(s0), "+v"(s1));
      if (!FIRST) settle(acc1, false, s1, mr1, l1);
      if (FIRST) l0 = s0;
      else settle(acc0, DIAG0, s0, mr0, l0);
      acc1 = acc1n;
      if (FIRST) mr1 = block_max(acc1, false);
      end(kb, steady_tag);
    };
    if (t0 == 0) {
      iter(0, T_{}, T_{}, St0{}, F_{});
    } else {
      iter(0, T_{}, F_{}, St0{}, F_{});
      int kb = 1;
      for (; kb + 2 < t0; kb += 3) {          // kb = 1 (mod 3); blocks up to kb + 4 <= t1 exist
        iter(kb, F_{}, F_{}, St1{}, T_{});
        iter(kb + 1, F_{}, F_{}, St2{}, T_{});
        iter(kb + 2, F_{}, F_{}, St0{}, T_{});
      }
      for (; kb < t0; ++kb) on_stage(kb, [&](auto st) __attribute__((always_inline)) { iter(kb, F_{}, F_{}, st, F_{}); });
      on_stage(t0, [&](auto st) __attribute__((always_inline)) { iter(t0, F_{}, T_{}, st, F_{}); });
    }
    on_stage(t1, [&](auto st) __attribute__((always_inline)) { read_k(st, ka); });
    const f32x16 acc1n = chain(ka, qb1);
    const float s1 = terms(acc1, false, mr1);
    settle(acc1, false, s1, mr1, l1);
    const float s1n = terms(acc1n, true, mr1);
    settle(acc1n, true, s1n, mr1, l1);
  } else {
    for (int kb = 0; kb <= t0; ++kb) {
      on_stage(kb, [&](auto st) __attribute__((always_inline)) {
        begin(kb, st, F_{});
        read_k(st, ka);
      });
      const f32x16 acc0 = chain(ka, qb0);
      const bool diag = kb == t0;
      if (kb == 0) {
        mr0 = block_max(acc0, diag);
        l0 = terms(acc0, diag, mr0);
      } else {
        settle(acc0, diag, terms(acc0, diag, mr0), mr0, l0);
      }
      if (kb < t0) end(kb, F_{});
    }
  }
  // merge the two lane halves (different keys of the same query row);
  // a half whose keys were all masked has l = 0
  auto finish = [&](float m, float l, int t) __attribute__((always_inline)) {
    const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
    const float M = fmaxf(l > 0.f ? m : kNegInf, l2 > 0.f ? m2 : kNegInf);
    const float L = (l > 0.f ? l * exp2_fast(m - M) : 0.f) + (l2 > 0.f ? l2 * exp2_fast(m2 - M) : 0.f);
    if (hh == 0) a.lse[lse_off + kTile * t + n32] = M + log2f(L);
  };
  finish(mr0, l0, t0);
  if (has1) finish(mr1, l1, t1);
}

// ------------------------------------------------------------------ pass 2: pooled scores

// One workgroup = tiles (t0 = 2p, t1 = 2p+1) of one KV head. For every staged
// key block before a tile, each wave (query head) forms S = Q.K^T, the
// probabilities exp2(s - lse_row), their sum over the tile's 32 rows; the G
// waves' sums are added through LDS (double-buffered, one barrier per block).
// Unless the rows change afterwards (pooling over all heads), the writer
// lanes also histogram the first digit (bits 31..21) of every pooled score
// they write, and at the end the workgroup finds each tile's bin of the k-th
// largest for the select (sel_pre), which then skips its histogram pass.
template <int D, int G, int OP = 0, typename E = __bf16>
__global__ __launch_bounds__(64 * G, 2) void pre_pool_kernel(PrefillArgs a) {
  constexpr int KC = D / 16;
  using KD = KDma<D, G>;
  // three K stages, filled two blocks ahead (as in the statistics pass)
  __shared__ __align__(1024) char s_k0[KD::BLKB];
  __shared__ __align__(1024) char s_k1[KD::BLKB];
  __shared__ __align__(1024) char s_k2[KD::BLKB];
  __shared__ float s_col[2][2][G][64];
  // first-digit histograms of the two tiles' pooled rows (G >= 4: with one or
  // two waves per workgroup their LDS would cost a wave per SIMD; the select
  // kernel histograms those rows itself)
  constexpr bool HIST = G >= 4;
  __shared__ uint32_t s_h1[HIST ? 2 : 1][HIST ? kBins1 : 1];
  __shared__ uint32_t s_tmp[G];
  __shared__ int s_res[2];
  const int pa0 = a.t_begin / 2;
  const int npairs = (a.t_end + 1) / 2 - pa0;
  const WorkItem it = work_item(blockIdx.x, npairs, a.Hkv, a.Hkv * a.B, true);
  const int p = pa0 + npairs - 1 - it.i;
  const int g = it.g, b = it.b;
  const int t0 = 2 * p, t1 = 2 * p + 1;
  const int Tb = tiles_of(a, b);
  if (t0 >= Tb) return;                           // past the sequence (whole workgroup)
  const bool has1 = t1 < Tb;
  const int nkb = has1 ? t1 : t0;              // key blocks before the later tile
  if (nkb == 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n32 = lane & 31, hh = lane >> 5;
  const int h = g * G + w;
  const int64_t lse_off = ((int64_t)b * a.Hq + h) * a.N;   // row statistics of this head
  // cleared before the first block's end barrier, whose wait covers LDS stores;
  // every histogram update comes after that barrier
  const bool hist = HIST && a.sel_pre != nullptr;
  if constexpr (HIST)
    if (hist)
      for (int i = threadIdx.x; i < 2 * kBins1; i += 64 * G) (&s_h1[0][0])[i] = 0u;
  u32x4 qa0[KC], qa1[KC];
  float lse0[16], lse1[16];
  {
    const int tq1 = has1 ? t1 : t0;
    const E* qh = (const E*)a.q + b * a.q_bstride + h * a.q_hstride;
    const E* q0 = qh + (int64_t)(kTile * t0 + n32) * a.q_tstride;
    const E* q1 = qh + (int64_t)(kTile * tq1 + n32) * a.q_tstride;
#pragma unroll
    for (int c = 0; c < KC; ++c) { qa0[c] = ldg16(q0 + 16 * c + 8 * hh); qa1[c] = ldg16(q1 + 16 * c + 8 * hh); }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      lse0[r] = a.lse[lse_off + kTile * t0 + mrow(r, hh)];
      lse1[r] = a.lse[lse_off + kTile * tq1 + mrow(r, hh)];
    }
  }
  const E* kbase = (const E*)a.k + b * a.kv_bstride + g * a.kv_hstride;
  float* out0 = a.pooled + pool_slot(a, b, g, t0);
  float* out1 = has1 ? a.pooled + pool_slot(a, b, g, t1) : out0;
  const float cs = a.scale_log2;
  KD kd;
  kd.init(kbase, a.N);
  auto chain = [&](const u32x4* ka, const u32x4* qa) __attribute__((always_inline)) {
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) acc = Ew<E>::mfma32(qa[c], ka[c], acc);   // S[query][key]
    return acc;
  };
  auto stage = [&](auto st_tag) __attribute__((always_inline)) -> char* {
    constexpr int ST = decltype(st_tag)::value;
    return ST == 0 ? s_k0 : (ST == 1 ? s_k1 : s_k2);
  };
  auto read_k = [&](auto st_tag, u32x4* ka) __attribute__((always_inline)) {
    const char* sk = stage(st_tag);
#pragma unroll
    for (int c = 0; c < KC; ++c) ka[c] = KD::read(sk, n32, 2 * c + hh);
  };
  // Column sums (OP 1: maxima) of one tile-block over the wave's 32 query
  // rows; both lane halves store their (equal) copy, so no lane branch splits
  // the block.
  auto pool = [](float x, float p) __attribute__((always_inline)) { return OP ? fmaxf(x, p) : x + p; };
  auto pool_halves = [](float x) __attribute__((always_inline)) { return OP ? xor32_max(x) : xor32_add(x); };
  auto colsum = [&](const f32x16& acc, const float* lse, float* dst) __attribute__((always_inline)) {
    float col = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) col = pool(col, exp2_fast(fmaf(acc[r], cs, -lse[r])));
    col = pool_halves(col);
    dst[lane] = col;
  };
  // An MFMA chain with the probability terms of an earlier, independent
  // block woven in (16 / KC after each MFMA, pinned by scheduling barriers),
  // then that block's column sums stored.
  auto chain_cols = [&](const u32x4* ka, const u32x4* qa, const f32x16& prev, const float* lse,
                        float* dst) __attribute__((always_inline)) {
    constexpr int TPM = 16 / KC;
    f32x16 acc = {};
    float col = 0.f;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
#pragma unroll
      for (int e = 0; e < TPM; ++e) col = pool(col, exp2_fast(fmaf(prev[TPM * c + e], cs, -lse[TPM * c + e])));
      acc = Ew<E>::mfma32(qa[c], ka[c], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    col = pool_halves(col);
    dst[lane] = col;
    return acc;
  };
  // Block kb is in stage kb % 3 (ST): the DMA of block kb + 2 before its
  // math, and after it block kb + 1 landed and the column sums in LDS, then
  // a barrier without a fence (STEADY: block kb + 2 exists).
  auto begin = [&](int kb, auto st_tag, auto steady_tag) __attribute__((always_inline)) {
    using S2 = std::integral_constant<int, (decltype(st_tag)::value + 2) % 3>;
    if (decltype(steady_tag)::value || kb + 2 < nkb) kd.issue(kTile * (kb + 2), stage(S2{}));
  };
  auto end = [&](int kb, auto steady_tag) __attribute__((always_inline)) {
    if (KD::EVEN && (decltype(steady_tag)::value || kb + 2 < nkb))
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(KD::NIW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_lgkm0_imm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2 = std::integral_constant<int, 2>;
  auto on_stage = [&](int kb, auto&& fn) __attribute__((always_inline)) {
    const int st = kb % 3;
    if (st == 0) fn(St0{});
    else if (st == 1) fn(St1{});
    else fn(St2{});
  };
  // Pool the G heads' column sums (maxima) of (tile, block) and write them out.
  auto emit = [&](int tile, int kb, int writer_wave) __attribute__((always_inline)) {
    if (w == writer_wave && hh == 0) {
      float sum = 0.f;
#pragma unroll
      for (int x = 0; x < G; ++x) sum = pool(sum, s_col[kb & 1][tile][x][n32]);
      (tile == 0 ? out0 : out1)[kTile * kb + n32] = sum;
      if constexpr (HIST)
        if (hist) atomicAdd(&s_h1[tile][__float_as_uint(sum) >> 21], 1u);
    }
  };
  const int w1 = G > 1 ? 1 : 0;
  kd.issue(0, s_k0);
  if (nkb > 1) kd.issue(kTile, s_k1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  u32x4 ka[KC];
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (has1) {
    f32x16 acc1 = {};
    auto iter = [&](int kb, auto first_tag, auto st_tag, auto steady_tag) __attribute__((always_inline)) {
      constexpr bool FIRST = decltype(first_tag)::value;
      begin(kb, st_tag, steady_tag);
      read_k(st_tag, ka);
      const f32x16 acc0 = FIRST ? chain(ka, qa0) : chain_cols(ka, qa0, acc1, lse1, s_col[(kb - 1) & 1][1][w]);
      acc1 = chain_cols(ka, qa1, acc0, lse0, s_col[kb & 1][0][w]);
      end(kb, steady_tag);
      emit(0, kb, 0);
      if (!FIRST) emit(1, kb - 1, w1);
    };
    if (t0 > 0) {
      iter(0, T_{}, St0{}, F_{});
      int kb = 1;
      for (; kb + 3 < t0; kb += 3) {          // kb = 1 (mod 3); blocks up to kb + 4 <= t0 exist
        iter(kb, F_{}, St1{}, T_{});
        iter(kb + 1, F_{}, St2{}, T_{});
        iter(kb + 2, F_{}, St0{}, T_{});
      }
      for (; kb < t0; ++kb) on_stage(kb, [&](auto st) __attribute__((always_inline)) { iter(kb, F_{}, st, F_{}); });
    }
    // block t0 is a candidate of tile 1 only
    on_stage(t0, [&](auto st) __attribute__((always_inline)) { read_k(st, ka); });
    const f32x16 acc1n = chain(ka, qa1);
    if (t0 > 0) colsum(acc1, lse1, s_col[(t0 - 1) & 1][1][w]);
    colsum(acc1n, lse1, s_col[t0 & 1][1][w]);
    __syncthreads();
    if (t0 > 0) emit(1, t0 - 1, w1);
    emit(1, t0, w1);
  } else {
    for (int kb = 0; kb < t0; ++kb) {
      on_stage(kb, [&](auto st) __attribute__((always_inline)) {
        begin(kb, st, F_{});
        read_k(st, ka);
      });
      const f32x16 acc0 = chain(ka, qa0);
      colsum(acc0, lse0, s_col[kb & 1][0][w]);
      end(kb, F_{});
      emit(0, kb, 0);
    }
  }
  // each tile's first-digit bin of the k-th largest pooled score, for the select
  if constexpr (HIST) if (hist) {
    __syncthreads();
    for (int tile = 0; tile < (has1 ? 2 : 1); ++tile) {
      const int t = tile ? t1 : t0;
      const uint32_t kt = (uint32_t)(a.offsets[t + 1] - a.offsets[t]);
      if (t >= 1 && kt > 0 && kt < (uint32_t)(kTile * t)) {   // uniform over the workgroup
        int b1;
        uint32_t ab1;
        block_find_bin_nt<64 * G>(s_h1[tile], kBins1, kt, s_tmp, s_res, b1, ab1);
        if (threadIdx.x == 0)
          reinterpret_cast<int4*>(a.sel_pre)[((int64_t)b * a.Hkv + g) * a.T + t] =
              int4{b1, (int)ab1, (int)s_h1[tile][b1], 0};
      }
    }
  }
}

// ------------------------------------------------------------------ pooling over all heads

// For one set per tile over all heads: the KV heads' pooled rows of (b, t)
// summed (OP 1: max) in KV-head order into KV head 0's row, in place. One
// workgroup per (tile, b); 16-byte accesses (rows are 128-byte aligned and
// 32 t long).
template <int OP>
__global__ __launch_bounds__(256) void pre_pool_heads_kernel(PrefillArgs a) {
  const int t = a.t_begin + blockIdx.x, b = blockIdx.y;
  if (t < 1 || t >= tiles_of(a, b)) return;
  const int n4 = kTile * t / 4;
  f32x4* dst = reinterpret_cast<f32x4*>(a.pooled + pool_slot(a, b, 0, t));
  for (int i = threadIdx.x; i < n4; i += 256) {
    f32x4 acc = dst[i];
    for (int g = 1; g < a.Hkv; ++g) {
      const f32x4 x = reinterpret_cast<const f32x4*>(a.pooled + pool_slot(a, b, g, t))[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = OP ? fmaxf(acc[e], x[e]) : acc[e] + x[e];
    }
    dst[i] = acc;
  }
}

// ------------------------------------------------------------------ Top-k per tile

// One workgroup per (tile, KV head): an exact radix select over the tile's
// pooled row (n = 32 t scores, rows 128-byte aligned, so every access is a
// whole 16-byte load): the bin of the k-th largest's first digit (bits
// 31..21), from the pooling pass (sel_pre) or a histogram pass over the row;
// the scores of that bin collected into LDS in a pass over the row, digits 2
// (bits 20..10) and 3 (bits 9..0) resolved there (a bin too large for LDS is
// histogrammed in two more passes over the row instead); a
// last pass writes the kept keys in index order (P > tau, then the first r
// keys equal to tau) through workgroup scans. Passes keep four 16-byte loads
// per thread in flight (indices past the row re-read its last vector and are
// not counted).
constexpr int kPreSelCap = 8192;   // LDS candidates of the k-th largest's first-digit bin
__global__ __launch_bounds__(256) void pre_select_kernel(PrefillArgs a) {
  __shared__ uint32_t s_h[kBins1];
  __shared__ uint32_t s_cand[kPreSelCap];
  __shared__ uint32_t s_tmp[4];
  __shared__ int s_res[2];
  __shared__ uint32_t s_nc;
  const WorkItem it = work_item(blockIdx.x, a.t_end - a.t_begin, a.Hsel, a.Hsel * a.B, true);
  const int t = a.t_end - 1 - it.i;
  const int g = it.g, b = it.b;
  if (t < 1 || t >= tiles_of(a, b)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = kTile * t;
  const int o0 = a.offsets[t];
  const uint32_t k = (uint32_t)(a.offsets[t + 1] - o0);
  if (k == 0) return;
  int32_t* out = a.idx_out + ((int64_t)b * a.Hsel + g) * a.total + o0;   // g < Hsel
  if (k >= (uint32_t)n) {
    for (int j = tid; j < n; j += 256) out[j] = j;
    return;
  }
  const uint32_t* P = reinterpret_cast<const uint32_t*>(a.pooled + pool_slot(a, b, g, t));
  const int n4 = n / 4;
  // fn(v, valid) on the 16-byte vectors g0 + tid + 256 q (q < 4) of each
  // group; every thread runs every group (the candidate appends use wave-wide
  // scans and shuffles), and indices past the row are loaded clamped and
  // passed as invalid
  auto pass = [&](auto&& fn) __attribute__((always_inline)) {
    for (int g0 = 0; g0 < n4; g0 += 4 * 256) {
      const int i0 = g0 + tid;
      u32x4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = ldg16(P + 4 * min(i0 + 256 * q, n4 - 1));
#pragma unroll
      for (int q = 0; q < 4; ++q) fn(v[q], i0 + 256 * q < n4);
    }
  };
  int b1, b2, b3;
  uint32_t ab1, ab2, ab3, nb1;
  if (a.sel_pre) {
    // the pooling pass histogrammed the row's first digit and found its bin
    const int4 pre = reinterpret_cast<const int4*>(a.sel_pre)[((int64_t)b * a.Hsel + g) * a.T + t];
    b1 = pre.x;
    ab1 = (uint32_t)pre.y;
    nb1 = (uint32_t)pre.z;
    for (int i = tid; i < kBins2; i += 256) s_h[i] = 0u;
    if (tid == 0) s_nc = 0u;
    __syncthreads();
  } else {
    for (int i = tid; i < kBins1; i += 256) s_h[i] = 0u;
    if (tid == 0) s_nc = 0u;
    __syncthreads();
    pass([&](const u32x4& v, bool ok) __attribute__((always_inline)) {
      if (ok) {
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(&s_h[v[e] >> 21], 1u);
      }
    });
    __syncthreads();
    block_find_bin(s_h, kBins1, k, s_tmp, s_res, b1, ab1);
    nb1 = s_h[b1];
    __syncthreads();
    for (int i = tid; i < kBins2; i += 256) s_h[i] = 0u;
    __syncthreads();
  }
  if (nb1 <= (uint32_t)a.sel_cap) {
    // the bin's scores into LDS (wave-aggregated appends), digits 2 and 3 there
    pass([&](const u32x4& v, bool ok) __attribute__((always_inline)) {
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c += (ok && (v[e] >> 21) == (uint32_t)b1) ? 1u : 0u;
      const uint32_t inc = wave_incl_scan_u32(c);
      uint32_t wbase = 0;
      if (lane == 63 && inc) wbase = atomicAdd(&s_nc, inc);
      wbase = __shfl(wbase, 63);
      uint32_t pos = wbase + inc - c;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ok && (v[e] >> 21) == (uint32_t)b1) s_cand[pos++] = v[e];
    });
    __syncthreads();
    for (uint32_t i = tid; i < nb1; i += 256) atomicAdd(&s_h[(s_cand[i] >> 10) & 0x7ffu], 1u);
    __syncthreads();
    block_find_bin(s_h, kBins2, k - ab1, s_tmp, s_res, b2, ab2);
    for (int i = tid; i < kBins3; i += 256) s_h[i] = 0u;
    __syncthreads();
    const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
    for (uint32_t i = tid; i < nb1; i += 256)
      if ((s_cand[i] >> 10) == pre) atomicAdd(&s_h[s_cand[i] & 0x3ffu], 1u);
    __syncthreads();
    block_find_bin(s_h, kBins3, k - ab1 - ab2, s_tmp, s_res, b3, ab3);
  } else {
    pass([&](const u32x4& v, bool ok) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ok && (v[e] >> 21) == (uint32_t)b1) atomicAdd(&s_h[(v[e] >> 10) & 0x7ffu], 1u);
    });
    __syncthreads();
    block_find_bin(s_h, kBins2, k - ab1, s_tmp, s_res, b2, ab2);
    for (int i = tid; i < kBins3; i += 256) s_h[i] = 0u;
    __syncthreads();
    const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
    pass([&](const u32x4& v, bool ok) __attribute__((always_inline)) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (ok && (v[e] >> 10) == pre) atomicAdd(&s_h[v[e] & 0x3ffu], 1u);
    });
    __syncthreads();
    block_find_bin(s_h, kBins3, k - ab1 - ab2, s_tmp, s_res, b3, ab3);
  }
  const uint32_t tau = (((uint32_t)b1 << 11 | (uint32_t)b2) << 10) | (uint32_t)b3;
  const uint32_t r = k - ab1 - ab2 - ab3;
  // stable compaction, 16 consecutive keys per thread per 4096-key chunk
  // (n is a multiple of 32, so a thread's 16 keys are all in or all out)
  constexpr int PER = 16;
  uint32_t gt_run = 0, eq_run = 0;
  for (int base = 0; base < n; base += 256 * PER) {
    const int j0 = base + tid * PER;
    const bool in = j0 < n;
    uint32_t u[PER];
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const u32x4 v = ldg16(P + min(j0, n - PER) + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * q + e] = v[e];
    }
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      gt += (in && u[i] > tau) ? 1u : 0u;
      eq += (in && u[i] == tau) ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan_256((gt << 16) | eq, s_tmp, &tot);   // both below 2^16 per chunk
    uint32_t g_ex = (ex >> 16) + gt_run;
    uint32_t e_ex = (ex & 0xffffu) + eq_run;
    if (in) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        if (u[i] > tau) {
          const uint32_t pos = g_ex + min(e_ex, r);
          if (pos < k) out[pos] = j0 + i;
          ++g_ex;
        } else if (u[i] == tau) {
          if (e_ex < r && g_ex + e_ex < k) out[g_ex + e_ex] = j0 + i;
          ++e_ex;
        }
      }
    }
    gt_run += tot >> 16;
    eq_run += tot & 0xffffu;
  }
}

// ------------------------------------------------------------------ sparse tile attention

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// gfx950 transposing LDS read (ds_read_b64_tr_b16). Within each group of 16
// lanes, source lane j supplies the address of 4 consecutive 16-bit values;
// lane i receives value i%4 of source lanes i/4, i/4+4, i/4+8, i/4+12
// (verified on the device with an index-grid probe).
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p)));
}

// ------------------------------------------------------------------ tile attention, LDS-DMA gathers


// Sparse tile attention: one workgroup per (query tile, KV head, batch), one
// wave per query head of the group (32 query rows each). The tile attends to
// its selected keys (the anchor's index set for the tile, 32 keys per block)
// and then to its own 32 keys under the causal mask (the diagonal block).
// Per block and wave: S^T = K.Q^T on eight 32x32x16 MFMAs (K rows from LDS,
// Q in registers), an online softmax, O += P.V on eight more MFMAs (V read
// from LDS by transposing reads); at the end O / l in the element type.
// The gathered K and V rows go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds: each lane names its own row chunk, the data
// lands at a fixed slot of a 1 KB line) through a ring of four stages, three
// blocks ahead of the math, so no registers hold rows in flight. The stages
// are distinct arrays selected at compile time (the steady loop is unrolled
// by four), so the compiler can tell the stage being read from the stages
// being filled.
// DENSE: dense causal attention with the same block math; block blk holds
// keys [32 blk, 32 blk + 32) for every blk <= t (block t is the diagonal), so
// there are no index loads and the tile's key list is [0, 32 t).
template <int D, int G, bool DENSE = false, typename E = __bf16>
__global__ __launch_bounds__(64 * G, 2) void pre_attn_dma_kernel(PrefillArgs a) {
  constexpr int NT = 64 * G, KC = D / 16, NDC = D / 32, PARTS = D / 8;
  constexpr int ROWB = 2 * D;               // bytes per row
  constexpr int BLKB = 32 * ROWB;           // one block of K (or V) rows
  constexpr int RPI = 64 / PARTS;           // rows per 1 KB DMA line
  constexpr int NINS = 32 / RPI;            // lines per block per tensor
  constexpr int NIW = (NINS + G - 1) / G;   // lines per wave (w, w + G, ...)
  constexpr bool EVEN = NINS % G == 0;      // every wave issues NIW lines
  constexpr float kBigP = Ew<E>::kBigP;     // half-row probability sum that triggers a rescale
  (void)NT;
  __shared__ __align__(1024) char s_st0[2 * BLKB];
  __shared__ __align__(1024) char s_st1[2 * BLKB];
  __shared__ __align__(1024) char s_st2[2 * BLKB];
  __shared__ __align__(1024) char s_st3[2 * BLKB];

  // global order for shorter prompts only: at 4096 tiles per unit the
  // per-head order measured 2 % faster (cache locality) and its tail is short
  const WorkItem it = work_item(blockIdx.x, a.T, a.Hkv, a.Hkv * a.B, a.T < kAttnGlobalOrderTiles);
  const int t = a.T - 1 - it.i;
  const int g = it.g, b = it.b;
  if (t >= tiles_of(a, b)) return;                          // past the sequence (whole workgroup)
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS line bases stay scalar
  const int n32 = lane & 31, hh = lane >> 5;
  const int h = g * G + w;
  int ga = (!DENSE && a.head_map) ? a.head_map[g] : g;
  ga = ((unsigned)ga < (unsigned)a.Hkv_a) ? ga : 0;
  const int o0 = DENSE ? 0 : a.offsets[t];
  const int kt = DENSE ? kTile * t : a.offsets[t + 1] - o0;
  const int32_t* S = DENSE ? nullptr : a.idx + ((int64_t)b * a.Hkv_a + ga) * a.total + o0;
  const int nsel = (kt + 31) / 32;
  const int nfull = kt / 32;
  const int tile_key0 = kTile * t;
  // Q fragments: B operand of S^T (lane: query n32, dims 16 c + 8 hh)
  u32x4 qf[KC];
  {
    const E* qrow = (const E*)a.q + b * a.q_bstride + h * a.q_hstride + (int64_t)(tile_key0 + n32) * a.q_tstride;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf[c] = ldg16(qrow + 16 * c + 8 * hh);
  }
  // K and V rows of this (b, g) through buffer resources: 32-bit row offsets,
  // and the buffer unit returns zeros for any offset past the N rows
  const E* kbase = (const E*)a.k + b * a.kv_bstride + (a.kvdiv > 1 ? g / a.kvdiv : g) * a.kv_hstride;
  const E* vbase = (const E*)a.v + b * a.kv_bstride + (a.kvdiv > 1 ? g / a.kvdiv : g) * a.kv_hstride;
  const int nbytes = (int)((int64_t)a.N * ROWB);
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, nbytes, kBufWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, nbytes, kBufWord3);
  const float cs = a.scale_log2;
  const int lrow = lane / PARTS, lslot = lane % PARTS;   // this lane's row / slot in a DMA line

  // raw indices of this lane's rows in the wave's lines of block blk (set blk %
  // 3), through a buffer resource over the tile's kt indices: positions past
  // the end read 0 (those rows belong to the partial block and are masked)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)S, (short)0, kt * 4, kBufWord3);
  int jr[4][NIW];
  auto load_index = [&](int blk, auto set_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    if constexpr (DENSE) return;
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int i = w + G * j;
      if (EVEN || i < NINS) {
        const int off = 4 * (blk * 32 + RPI * i + lrow);
        jr[SET][j] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
      }
    }
  };
  auto stage = [&](auto st_tag) __attribute__((always_inline)) -> char* {
    constexpr int ST = decltype(st_tag)::value;
    return ST == 0 ? s_st0 : (ST == 1 ? s_st1 : (ST == 2 ? s_st2 : s_st3));
  };
  // DMA the K and V rows of block blk into a stage (the causal diagonal block
  // nsel reads rows tile_key0 ..; padding rows read row 0 and are masked)
  // (STEADY: blk is a full selected block, so only the index range check remains)
  auto issue = [&](int blk, auto set_tag, char* dst, auto steady_tag) __attribute__((always_inline)) {
    constexpr int SET = decltype(set_tag)::value;
    constexpr bool STEADY = decltype(steady_tag)::value;
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
      const int i = w + G * j;
      if (EVEN || i < NINS) {
        const int r = RPI * i + lrow;
        int key;
        if constexpr (DENSE) {
          key = blk * 32 + r;                                    // blk <= t: inside the prompt
        } else {
          const int jj = jr[SET][j];
          if (STEADY) {
            key = ((unsigned)jj < (unsigned)tile_key0) ? jj : 0;   // trusted input, kept in bounds
          } else {
            const int sel = (blk * 32 + r < kt && (unsigned)jj < (unsigned)tile_key0) ? jj : 0;
            key = (blk == nsel) ? tile_key0 + r : sel;
          }
        }
        // byte offsets of the row plus this lane's swizzled 16-byte chunk
        // (computed before the call: a function call inside the builtin's
        // argument list makes the host pass drop the kernel's launch stub)
        const int koff = key * ROWB + 16 * (lslot ^ swz_k<D>(r));
        const int voff = key * ROWB + 16 * (lslot ^ swz_v<D>(r));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16,
                                                 koff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(dst + BLKB + 1024 * i),
                                                 16, voff, 0, 0, 0);
      }
    }
  };
  // P.V operand addressing (transposing read): lane group g16 = lane/16,
  // member j = lane%16 reads row 4*hh + j/4 (+8 for the upper keys), chunk
  // 4 dc + 2 (g16 % 2) + (j % 4) / 2, half (j % 4) % 2 of it.
  const int g16 = lane >> 4, j16 = lane & 15;
  const int tr_row = 4 * hh + (j16 >> 2);
  const int tr_q = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  const int tr_half = 8 * ((j16 & 3) & 1);

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) o[dc] = f32x16{};

  // One key block on stage ST = blk % 4 (MODE 0: full selected block; 1: the
  // partial last one; 2: the causal diagonal). Before the math: indices of
  // block blk + 4 (into set ST, free since block blk's lines were issued) and
  // the DMA of block blk + 3 (into stage (ST + 3) % 4, block blk - 1's,
  // released by the last barrier). After it: block blk + 1's lines complete in
  // every wave, then a barrier.
  auto step = [&](int blk, auto mode_tag, auto st_tag, auto steady_tag) __attribute__((always_inline)) {
    constexpr int MODE = decltype(mode_tag)::value;
    constexpr int ST = decltype(st_tag)::value;
    constexpr bool STEADY = decltype(steady_tag)::value;
    using SetN = std::integral_constant<int, ST>;             // (blk + 4) % 4
    using St2 = std::integral_constant<int, (ST + 3) % 4>;    // (blk + 3) % 4
    if (STEADY || blk + 4 < nsel) load_index(blk + 4, SetN{});
    // the indices of block blk + 3 (loaded a step ago, before block blk + 2's
    // lines and this step's index loads) have landed; said with the builtin
    // so the compiler does not wait for everything in flight before using them
    if (STEADY && EVEN && !DENSE) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * NIW));
    if (STEADY || blk + 3 <= nsel) issue(blk + 3, St2{}, stage(St2{}), steady_tag);
    const char* sk = stage(st_tag);
    const char* sv = sk + BLKB;
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 kk = *reinterpret_cast<const u32x4*>(sk + n32 * ROWB + 16 * ((2 * c + hh) ^ swz_k<D>(n32)));
      acc = Ew<E>::mfma32(kk, qf[c], acc);             // S^T[key slot][query]
    }
    if (MODE != 0) {
      const int nvalid = kt - blk * 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int slot = mrow(r, hh);
        const bool ok = (MODE == 2) ? (slot <= n32) : (slot < nvalid);
        acc[r] = ok ? acc[r] : kNegInf;
      }
    }
    // Online softmax with a lazy reference: m_run of a query row is the
    // maximum of its first block, and later blocks are exponentiated against
    // it without a maximum of their own. A row whose probabilities grow too
    // large for the accumulators (its half-row sum above 2^64, or not finite)
    // takes the rare path: the block maximum over both lane halves of the row,
    // o and l rescaled by 2^(m_run - m_new), the probabilities recomputed. The
    // reference cancels in o / l; it only has to keep the exponentials finite.
    // (alpha moves from the S^T layout, lane = query, to the output layout,
    // reg r = query mrow(r, hh), by shuffles.)
    if (blk == 0) m_run = xor32_max(max16(acc)) * cs;   // cs > 0
    u32x4 pa[2];
    float ps;
    auto probs = [&]() __attribute__((always_inline)) {
      ps = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = exp2_fast(fmaf(acc[8 * c2 + 2 * e], cs, -m_run));       // -inf -> 0
          const float p1 = exp2_fast(fmaf(acc[8 * c2 + 2 * e + 1], cs, -m_run));
          pa[c2][e] = Ew<E>::pack2(p0, p1);
          ps = Ew<E>::add2(pa[c2][e], ps);     // the row sum of the 16-bit weights P.V uses
        }
      }
    };
    probs();
    if (__builtin_expect(__any(!(ps <= kBigP)), 0)) {
      const float bm = xor32_max(max16(acc)) * cs;
      const bool bump = bm > m_run + 8.f;
      const float m_new = bump ? bm : m_run;
      const float alpha = exp2_fast(m_run - m_new);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float ar = __shfl(alpha, mrow(r, hh));
#pragma unroll
        for (int dc = 0; dc < NDC; ++dc) o[dc][r] *= ar;
      }
      l_run *= alpha;
      m_run = m_new;
      probs();
    }
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int R = 16 * c2 + tr_row;
      const int sw = swz_v<D>(R);                // rows R and R + 8 share it
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const int cofs = 16 * ((4 * dc + tr_q) ^ sw) + tr_half;
        const u32x2 lo = lds_read_tr16(sv + R * ROWB + cofs);
        const u32x2 hi = lds_read_tr16(sv + (R + 8) * ROWB + cofs);
        const u32x4 vb = {lo[0], lo[1], hi[0], hi[1]};
        o[dc] = Ew<E>::mfma32(pa[c2], vb, o[dc]);
      }
    }
    l_run += ps;
    // block blk + 1 complete in this wave (steady: only the index loads and
    // DMA lines of this step and the last one may still be in flight), then
    // in every wave
    // (the builtin wait, unlike inline asm, is seen by the compiler's own
    // wait placement, which then knows these lines have landed; DENSE has no
    // index loads in flight, only the lines of blocks blk + 2 and blk + 3)
    if (STEADY && EVEN) {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(DENSE ? 4 * NIW : 6 * NIW));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  using St0 = std::integral_constant<int, 0>;
  using St1 = std::integral_constant<int, 1>;
  using St2c = std::integral_constant<int, 2>;
  using St3c = std::integral_constant<int, 3>;
  using Steady = std::true_type;
  using Tail = std::false_type;
  // prologue: indices of blocks 0..3, lines of blocks 0..2
  if (0 < nsel) load_index(0, St0{});
  if (1 < nsel) load_index(1, St1{});
  if (2 < nsel) load_index(2, St2c{});
  if (3 < nsel) load_index(3, St3c{});
  issue(0, St0{}, s_st0, std::false_type{});
  if (1 <= nsel) issue(1, St1{}, s_st1, std::false_type{});
  if (2 <= nsel) issue(2, St2c{}, s_st2, std::false_type{});
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  int blk = 0;
  // steady state: blocks blk .. blk + 3 full, indices of blk + 7 exist
  for (; blk + 7 < nsel; blk += 4) {
    step(blk, std::integral_constant<int, 0>{}, St0{}, Steady{});
    step(blk + 1, std::integral_constant<int, 0>{}, St1{}, Steady{});
    step(blk + 2, std::integral_constant<int, 0>{}, St2c{}, Steady{});
    step(blk + 3, std::integral_constant<int, 0>{}, St3c{}, Steady{});
  }
  auto step_any = [&](int bk, auto mode_tag) __attribute__((always_inline)) {
    const int st = bk & 3;
    if (st == 0) step(bk, mode_tag, St0{}, Tail{});
    else if (st == 1) step(bk, mode_tag, St1{}, Tail{});
    else if (st == 2) step(bk, mode_tag, St2c{}, Tail{});
    else step(bk, mode_tag, St3c{}, Tail{});
  };
  for (; blk < nfull; ++blk) step_any(blk, std::integral_constant<int, 0>{});
  if (nsel > nfull) step_any(nfull, std::integral_constant<int, 1>{});
  step_any(nsel, std::integral_constant<int, 2>{});
  // normalise: 1/l of query q lives in lane q; output rows are mrow(r, hh)
  const float inv_l = 1.0f / xor32_add(l_run);
  uint16_t* ob = reinterpret_cast<uint16_t*>(a.o) + b * a.o_bstride + h * a.o_hstride + (int64_t)tile_key0 * a.o_tstride;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float inv = __shfl(inv_l, mrow(r, hh));
#pragma unroll
    for (int dc = 0; dc < NDC; ++dc)
      ob[(int64_t)mrow(r, hh) * a.o_tstride + n32 + 32 * dc] = Ew<E>::bits(o[dc][r] * inv);
  }
}

// ------------------------------------------------------------------ paged caches

// One workgroup per (32-row tile, KV head, sequence): the tile's K and V rows,
// each found through the block table (page = id of entry row / P, row % P
// inside it), into the contiguous copies. Tiles past the prompt are skipped:
// the tile kernels read no key row at or past the prompt's last whole tile.
// 16 bytes per lane per load; D / 64 loads of K and as many of V in flight.
template <int D>
__global__ __launch_bounds__(256) void pre_page_copy_kernel(PageCopyArgs c) {
  constexpr int PARTS = D / 8;                    // 16-byte chunks per row
  constexpr int PER = kTile * PARTS / 256;        // chunks per lane per tensor
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if (t >= tiles_in(c.seq_lens, b, c.N, c.T)) return;
  const int32_t* bt = c.block_table + (int64_t)b * c.max_pages;
  const int64_t pmask = (int64_t(1) << c.shift) - 1;
  const uint16_t* ks = (const uint16_t*)c.k;
  const uint16_t* vs = (const uint16_t*)c.v;
  const int64_t dst0 = (((int64_t)b * c.Hkv + g) * c.N + (int64_t)t * kTile) * D;
  u32x4 kx[PER], vx[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = threadIdx.x + 256 * i, r = e / PARTS, part = e % PARTS;
    const int64_t row = (int64_t)t * kTile + r;       // < N, so row / P < max_pages
    int64_t page = bt[row >> c.shift];
    page = page < 0 ? 0 : (page >= c.num_pages ? c.num_pages - 1 : page);
    const int64_t src = page * c.page_stride + g * c.page_hstride + (row & pmask) * D + 8 * part;
    kx[i] = ldg16(ks + src);
    vx[i] = ldg16(vs + src);
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t dst = dst0 + (int64_t)(threadIdx.x + 256 * i) * 8;
    *reinterpret_cast<u32x4*>((uint16_t*)c.kc + dst) = kx[i];
    *reinterpret_cast<u32x4*>((uint16_t*)c.vc + dst) = vx[i];
  }
}

// ------------------------------------------------------------------ host side

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int64_t pool_budget_floats() {
  const int64_t v = option_value(KAS_OPT_PREFILL_POOL_MB);
  const int64_t mb = v > 0 ? v : kPoolBudgetMBDefault;
  return mb * (1 << 20) / 4;
}

// Tiles [ta, tb) per pool/select launch so that the pooled rows fit the budget.
// Chunks start at even tiles so that tile pairs (2p, 2p+1) never straddle two.
static int next_chunk_end(int ta, int T, int64_t units, int64_t budget) {
  int64_t used = 0;
  int tb = ta;
  while (tb < T) {
    const int64_t need = units * kTile * ((int64_t)tb + (tb + 1 < T ? tb + 1 : 0));
    if (tb > ta && used + need > budget) break;
    used += need;
    tb = (tb + 2 < T) ? tb + 2 : T;
  }
  return tb;
}

static int64_t max_chunk_floats(int T, int64_t units, int64_t budget) {
  int64_t best = 0;
  for (int ta = 0; ta < T;) {
    const int tb = next_chunk_end(ta, T, units, budget);
    const int64_t f = units * kTile * ((int64_t)tb * (tb - 1) / 2 - (int64_t)ta * (ta - 1) / 2);
    best = f > best ? f : best;
    ta = tb;
  }
  return best;
}

struct PrefillPlan {
  size_t off_offsets, off_lse, off_pooled, off_sel_pre, total;
  int64_t pooled_floats;
};

static PrefillPlan plan(int B, int Hq, int Hkv, int64_t N, bool anchor) {
  PrefillPlan p{};
  const int T = (int)(N / kTile);
  size_t off = 0;
  auto take = [&](size_t bytes) __attribute__((always_inline)) { size_t o = off; off = align256(off + bytes); return o; };
  p.off_offsets = take((size_t)(T + 1) * sizeof(int32_t));
  if (anchor) {
    p.off_lse = take((size_t)B * Hq * N * sizeof(float));
    p.pooled_floats = max_chunk_floats(T, (int64_t)B * Hkv, pool_budget_floats());
    p.off_pooled = take((size_t)(p.pooled_floats > 0 ? p.pooled_floats : 1) * sizeof(float));
    p.off_sel_pre = take((size_t)B * Hkv * T * 4 * sizeof(int32_t));
  }
  p.total = off;
  return p;
}

size_t prefill_workspace_bytes(int B, int Hq, int Hkv, int D, int64_t N, int pct, bool anchor) {
  (void)D; (void)pct;
  return plan(B, Hq, Hkv, N, anchor).total;
}

void fill_prefill_args(PrefillArgs& a, int B, int Hq, int Hkv, int D, int64_t N, int pct, float scale,
                       int64_t kv_bs, int64_t kv_hs, char* ws, bool anchor) {
  a = PrefillArgs{};
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.G = Hq / Hkv; a.N = N; a.pct = pct;
  a.T = (int)(N / kTile);
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.kv_bstride = kv_bs; a.kv_hstride = kv_hs;
  a.Hsel = Hkv;
  a.kvdiv = 1;
  PrefillPlan p = plan(B, Hq, Hkv, N, anchor);
  // the tuning option lowers the LDS candidate cap of the select (0 sends
  // every tile through the in-place histogram passes)
  const int64_t cap = option_value(KAS_OPT_PREFILL_SELECT_CAP);
  a.sel_cap = cap >= 0 ? (int)std::min<int64_t>(cap, kPreSelCap) : kPreSelCap;
  if (!ws) return;                  // dense attention: no workspace
  a.offsets = (int32_t*)(ws + p.off_offsets);
  if (anchor) {
    a.lse = (float*)(ws + p.off_lse);
    a.pooled = (float*)(ws + p.off_pooled);
    a.pooled_floats = (size_t)p.pooled_floats;
    a.sel_pre = (int32_t*)(ws + p.off_sel_pre);
  }
}

#define KAS_LAUNCH_P(kernel, grid, block, ctx, arg) (ctx).launch(kernel, grid, block, arg)

// fn(D, G, E) with head_dim D, group size G and element type E (tags whose
// ::value / type name them at compile time) for the supported shapes.
template <typename E>
struct ETag { using type = E; };
template <typename F>
static hipError_t for_dge(const PrefillArgs& a, F&& fn) {
  auto by_g = [&](auto dc, auto et) -> hipError_t {
    switch (a.G) {
      case 1: fn(dc, std::integral_constant<int, 1>{}, et); return hipSuccess;
      case 2: fn(dc, std::integral_constant<int, 2>{}, et); return hipSuccess;
      case 4: fn(dc, std::integral_constant<int, 4>{}, et); return hipSuccess;
      case 8: fn(dc, std::integral_constant<int, 8>{}, et); return hipSuccess;
    }
    return hipErrorInvalidValue;
  };
  auto by_d = [&](auto et) -> hipError_t {
    return a.D == 128 ? by_g(std::integral_constant<int, 128>{}, et) : by_g(std::integral_constant<int, 64>{}, et);
  };
  return a.dtype == 2 ? by_d(ETag<_Float16>{}) : by_d(ETag<__bf16>{});
}
#define KAS_DGE(dc, gc, et) \
  constexpr int D = decltype(dc)::value, G = decltype(gc)::value; using E = typename decltype(et)::type

// Work items of a one-dimensional grid (workgroup ids stay below 2^31).
static bool grid_fits(int64_t items) { return items > 0 && items < (int64_t(1) << 31); }

static hipError_t launch_offsets(PrefillArgs& a, LaunchCtx& ctx) {
  KAS_LAUNCH_P(pre_offsets_kernel, dim3(1), dim3(256), ctx, a);
  return hipGetLastError();
}

template <bool DENSE>
static hipError_t launch_tile_attn(PrefillArgs& a, LaunchCtx& ctx, int kid) {
  if (!grid_fits((int64_t)a.T * a.Hkv * a.B)) return hipErrorInvalidConfiguration;
  ctx.begin(kid);
  const dim3 grid((unsigned)((int64_t)a.T * a.Hkv * a.B));
  hipError_t e = for_dge(a, [&](auto dc, auto gc, auto et) {
    KAS_DGE(dc, gc, et);
    ctx.launch(pre_attn_dma_kernel<D, G, DENSE, E>, grid, dim3(64 * G), a);
  });
  if (e != hipSuccess) return e;
  return ctx.end(kid);
}

static hipError_t launch_attn(PrefillArgs& a, LaunchCtx& ctx) { return launch_tile_attn<false>(a, ctx, K_PRE_ATTN); }

hipError_t launch_prefill_dense(PrefillArgs& a, LaunchCtx& ctx) { return launch_tile_attn<true>(a, ctx, K_PRE_DENSE); }

hipError_t launch_prefill_anchor(PrefillArgs& a, LaunchCtx& ctx) {
  hipError_t e;
  // no first-digit bins from the pooling pass when the heads' rows are summed
  // after pooling, or for groups of fewer than 4 heads (see pre_pool_kernel)
  if (a.pool_all || a.G < 4) a.sel_pre = nullptr;
  if ((e = launch_offsets(a, ctx)) != hipSuccess) return e;
  if (!grid_fits((int64_t)((a.T + 1) / 2) * a.Hkv * a.B)) return hipErrorInvalidConfiguration;
  ctx.begin(K_PRE_STATS);
  {
    const dim3 grid((unsigned)((int64_t)((a.T + 1) / 2) * a.Hkv * a.B));
    e = for_dge(a, [&](auto dc, auto gc, auto et) {
      KAS_DGE(dc, gc, et);
      ctx.launch(pre_stats_kernel<D, G, E>, grid, dim3(64 * G), a);
    });
    if (e != hipSuccess) return e;
  }
  if ((e = ctx.end(K_PRE_STATS)) != hipSuccess) return e;
  const int64_t units = (int64_t)a.B * a.Hkv;
  const int64_t budget = pool_budget_floats();
  for (int ta = 0; ta < a.T;) {
    const int tb = next_chunk_end(ta, a.T, units, budget);
    a.t_begin = ta;
    a.t_end = tb;
    const dim3 pgrid((unsigned)((int64_t)((tb + 1) / 2 - ta / 2) * a.Hkv * a.B));
    ctx.begin(K_PRE_POOL);
    e = for_dge(a, [&](auto dc, auto gc, auto et) {
      KAS_DGE(dc, gc, et);
      if (a.pool_op) ctx.launch(pre_pool_kernel<D, G, 1, E>, pgrid, dim3(64 * G), a);
      else ctx.launch(pre_pool_kernel<D, G, 0, E>, pgrid, dim3(64 * G), a);
    });
    if (e != hipSuccess) return e;
    if ((e = ctx.end(K_PRE_POOL)) != hipSuccess) return e;
    if (a.pool_all) {
      ctx.begin(K_PRE_POOL_HEADS);
      if (a.pool_op) KAS_LAUNCH_P(pre_pool_heads_kernel<1>, dim3(tb - ta, a.B), dim3(256), ctx, a);
      else KAS_LAUNCH_P(pre_pool_heads_kernel<0>, dim3(tb - ta, a.B), dim3(256), ctx, a);
      if ((e = ctx.end(K_PRE_POOL_HEADS)) != hipSuccess) return e;
    }
    dim3 grid((unsigned)((int64_t)(tb - ta) * a.Hsel * a.B));
    ctx.begin(K_PRE_SELECT);
    KAS_LAUNCH_P(pre_select_kernel, grid, dim3(256), ctx, a);
    if ((e = ctx.end(K_PRE_SELECT)) != hipSuccess) return e;
    ta = tb;
  }
  return a.dense_out ? launch_prefill_dense(a, ctx) : launch_attn(a, ctx);
}

hipError_t launch_prefill_page_copy(const PageCopyArgs& c, LaunchCtx& ctx) {
  ctx.begin(K_PRE_PAGE_COPY);
  const dim3 grid(c.T, c.Hkv, c.B);
  if (c.D == 128) ctx.launch(pre_page_copy_kernel<128>, grid, dim3(256), c);
  else ctx.launch(pre_page_copy_kernel<64>, grid, dim3(256), c);
  return ctx.end(K_PRE_PAGE_COPY);
}

hipError_t launch_prefill_reuse(PrefillArgs& a, LaunchCtx& ctx) {
  hipError_t e;
  if ((e = launch_offsets(a, ctx)) != hipSuccess) return e;
  return launch_attn(a, ctx);
}

}  // namespace kas
