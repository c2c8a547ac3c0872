// Prefill-phase kernels for gfx950: query tiles of 32 rows, bf16 inputs,
// 32x32x16 bf16 MFMA tiles, fp32 softmax.
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
//               the fp32 bit pattern, ties to the lower index), written as
//               ascending CSR indices.
//  pre_attn     anchor output and reuse layers: one workgroup per (tile, KV
//               head), gathered K rows and transposed V rows in LDS, S^T and
//               P.V on MFMA, online softmax over the tile's index set plus
//               its causal diagonal block.
#include "kas_block.hpp"
#include "kas_prefill.hpp"

namespace kas {

constexpr int kPoolBudgetMBDefault = 2048;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

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

// ------------------------------------------------------------------ K tile staging

// 32 consecutive (or gathered) K rows -> LDS, row stride KROW bytes.
template <int D, int NT>
__device__ __forceinline__ void stage_k_rows(char* s_k, int krow_bytes, const __bf16* kbase,
                                             const int* rows /* nullptr: contiguous from row0 */,
                                             int64_t row0) {
  constexpr int PARTS = D / 8;
  for (int x = threadIdx.x; x < 32 * PARTS; x += NT) {
    const int r = x / PARTS, part = x % PARTS;
    const int64_t src = rows ? (int64_t)rows[r] : row0 + r;
    *reinterpret_cast<u32x4*>(s_k + r * krow_bytes + part * 16) = ldg16(kbase + src * D + part * 8);
  }
}

// ------------------------------------------------------------------ pass 1: row statistics

template <int D, int G>
__global__ __launch_bounds__(64 * G) void pre_stats_kernel(PrefillArgs a) {
  constexpr int NT = 64 * G, KC = D / 16, KROW = 2 * D + 16;
  __shared__ __align__(16) char s_k[32 * KROW];
  const int t = a.T - 1 - blockIdx.x;          // long rows first
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n32 = lane & 31, hh = lane >> 5;
  const int h = g * G + w;
  const __bf16* qrow = (const __bf16*)a.q + (((int64_t)b * a.Hq + h) * a.N + kTile * t + n32) * D;
  u32x4 qb[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) qb[c] = ldg16(qrow + 16 * c + 8 * hh);
  const __bf16* kbase = (const __bf16*)a.k + b * a.kv_bstride + g * a.kv_hstride;
  const float cs = a.scale_log2;
  float m = kNegInf, l = 0.f;
  for (int kb = 0; kb <= t; ++kb) {
    __syncthreads();
    stage_k_rows<D, NT>(s_k, KROW, kbase, nullptr, (int64_t)kTile * kb);
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(s_k + n32 * KROW + (16 * c + 8 * hh) * 2);
      acc = mfma32(ka, qb[c], acc);             // S^T[key][query]
    }
    if (kb == t) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (mrow(r, hh) > n32) acc[r] = kNegInf;
    }
    float bm = acc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) bm = fmaxf(bm, acc[r]);
    const float mn = fmaxf(m, bm * cs);
    if (mn != kNegInf) {
      const float al = (mn == m) ? 1.f : exp2_fast(m - mn);
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) s += exp2_fast(fmaf(acc[r], cs, -mn));
      l = l * al + s;
      m = mn;
    }
  }
  const float m2 = __shfl_xor(m, 32), l2 = __shfl_xor(l, 32);
  const float M = fmaxf(m, m2);
  const float L = (m == kNegInf ? 0.f : l * exp2_fast(m - M)) + (m2 == kNegInf ? 0.f : l2 * exp2_fast(m2 - M));
  if (hh == 0) a.lse[((int64_t)b * a.Hq + h) * a.N + kTile * t + n32] = M + log2f(L);
}

// ------------------------------------------------------------------ pass 2: pooled scores

template <int D, int G>
__global__ __launch_bounds__(64 * G) void pre_pool_kernel(PrefillArgs a) {
  constexpr int NT = 64 * G, KC = D / 16, KROW = 2 * D + 16;
  __shared__ __align__(16) char s_k[32 * KROW];
  __shared__ float s_col[G][32];
  const int t = a.t_end - 1 - blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  if (t < 1) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n32 = lane & 31, hh = lane >> 5;
  const int h = g * G + w;
  const int64_t qoff = ((int64_t)b * a.Hq + h) * a.N + kTile * t;
  const __bf16* qrow = (const __bf16*)a.q + (qoff + n32) * D;
  u32x4 qa[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) qa[c] = ldg16(qrow + 16 * c + 8 * hh);
  float lse[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) lse[r] = a.lse[qoff + mrow(r, hh)];
  const __bf16* kbase = (const __bf16*)a.k + b * a.kv_bstride + g * a.kv_hstride;
  float* out = a.pooled + pool_slot(a, b, g, t);
  const float cs = a.scale_log2;
  for (int kb = 0; kb < t; ++kb) {
    __syncthreads();
    stage_k_rows<D, NT>(s_k, KROW, kbase, nullptr, (int64_t)kTile * kb);
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 kbv = *reinterpret_cast<const u32x4*>(s_k + n32 * KROW + (16 * c + 8 * hh) * 2);
      acc = mfma32(qa[c], kbv, acc);            // S[query][key]
    }
    float col = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) col += exp2_fast(fmaf(acc[r], cs, -lse[r]));
    col += __shfl_xor(col, 32);
    if (hh == 0) s_col[w][n32] = col;
    __syncthreads();
    if (w == 0 && hh == 0) {
      float s = 0.f;
#pragma unroll
      for (int x = 0; x < G; ++x) s += s_col[x][n32];
      out[kTile * kb + n32] = s;
    }
  }
}

// ------------------------------------------------------------------ Top-k per tile

__global__ __launch_bounds__(256) void pre_select_kernel(PrefillArgs a) {
  __shared__ uint32_t s_h[kBins1];
  __shared__ uint32_t s_tmp[4];
  __shared__ int s_res[2];
  const int t = a.t_end - 1 - blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  if (t < 1) return;
  const int tid = threadIdx.x;
  const int n = kTile * t;
  const int o0 = a.offsets[t];
  const uint32_t k = (uint32_t)(a.offsets[t + 1] - o0);
  if (k == 0) return;
  int32_t* out = a.idx_out + ((int64_t)b * a.Hkv + g) * a.total + o0;
  if (k >= (uint32_t)n) {
    for (int j = tid; j < n; j += 256) out[j] = j;
    return;
  }
  const uint32_t* P = reinterpret_cast<const uint32_t*>(a.pooled + pool_slot(a, b, g, t));
  // digit 1
  for (int i = tid; i < kBins1; i += 256) s_h[i] = 0u;
  __syncthreads();
  for (int j = tid; j < n; j += 256) atomicAdd(&s_h[P[j] >> 21], 1u);
  __syncthreads();
  int b1, b2, b3;
  uint32_t ab1, ab2, ab3;
  block_find_bin(s_h, kBins1, k, s_tmp, s_res, b1, ab1);
  // digit 2
  for (int i = tid; i < kBins2; i += 256) s_h[i] = 0u;
  __syncthreads();
  for (int j = tid; j < n; j += 256) {
    const uint32_t u = P[j];
    if ((u >> 21) == (uint32_t)b1) atomicAdd(&s_h[(u >> 10) & 0x7ffu], 1u);
  }
  __syncthreads();
  block_find_bin(s_h, kBins2, k - ab1, s_tmp, s_res, b2, ab2);
  // digit 3
  for (int i = tid; i < kBins3; i += 256) s_h[i] = 0u;
  __syncthreads();
  const uint32_t pre = ((uint32_t)b1 << 11) | (uint32_t)b2;
  for (int j = tid; j < n; j += 256) {
    const uint32_t u = P[j];
    if ((u >> 10) == pre) atomicAdd(&s_h[u & 0x3ffu], 1u);
  }
  __syncthreads();
  block_find_bin(s_h, kBins3, k - ab1 - ab2, s_tmp, s_res, b3, ab3);
  const uint32_t tau = (pre << 10) | (uint32_t)b3;
  const uint32_t r = k - ab1 - ab2 - ab3;
  // stable compaction, 16 consecutive keys per thread per 4096-key chunk
  constexpr int PER = 16;
  uint32_t gt_run = 0, eq_run = 0;
  for (int base = 0; base < n; base += 256 * PER) {
    const int j0 = base + tid * PER;
    uint32_t u[PER];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool in = j0 + i < n;
      u[i] = in ? P[j0 + i] : 0u;
      gt += in && u[i] > tau;
      eq += in && u[i] == tau;
    }
    uint32_t tg, te;
    uint32_t g_ex = block_excl_scan_256(gt, s_tmp, &tg) + gt_run;
    uint32_t e_ex = block_excl_scan_256(eq, s_tmp, &te) + eq_run;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (j0 + i >= n) break;
      if (u[i] > tau) {
        const uint32_t pos = g_ex + min(e_ex, r);
        if (pos < k) out[pos] = j0 + i;
        ++g_ex;
      } else if (u[i] == tau) {
        if (e_ex < r && g_ex + e_ex < k) out[g_ex + e_ex] = j0 + i;
        ++e_ex;
      }
    }
    gt_run += tg;
    eq_run += te;
  }
}

// ------------------------------------------------------------------ sparse tile attention

template <int D, int G>
__global__ __launch_bounds__(64 * G) void pre_attn_kernel(PrefillArgs a) {
  constexpr int NT = 64 * G, KC = D / 16, NDC = D / 32;
  constexpr int KROW = 2 * D + 16;   // bytes per K row in LDS
  constexpr int VROW = 2 * 32 + 8;   // bytes per V^T row (32 keys + pad)
  __shared__ __align__(16) char s_k[32 * KROW];
  __shared__ __align__(16) char s_vt[D * VROW];
  __shared__ int s_key[32];
  __shared__ float s_x[G][32];

  const int t = a.T - 1 - blockIdx.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n32 = lane & 31, hh = lane >> 5;
  const int h = g * G + w;
  int ga = a.head_map ? a.head_map[g] : g;
  ga = ((unsigned)ga < (unsigned)a.Hkv_a) ? ga : 0;
  const int o0 = a.offsets[t];
  const int kt = a.offsets[t + 1] - o0;
  const int32_t* S = a.idx + ((int64_t)b * a.Hkv_a + ga) * a.total + o0;
  const int nsel = (kt + 31) / 32;

  const int64_t qoff = ((int64_t)b * a.Hq + h) * a.N + kTile * t;
  u32x4 qb[KC];
  {
    const __bf16* qrow = (const __bf16*)a.q + (qoff + n32) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) qb[c] = ldg16(qrow + 16 * c + 8 * hh);
  }
  const __bf16* kbase = (const __bf16*)a.k + b * a.kv_bstride + g * a.kv_hstride;
  const __bf16* vbase = (const __bf16*)a.v + b * a.kv_bstride + g * a.kv_hstride;
  const float cs = a.scale_log2;
  const int tile_key0 = kTile * t;

  float m_run = kNegInf, l_run = 0.f;
  f32x16 o[NDC];
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc) o[dc] = f32x16{};

  for (int blk = 0; blk <= nsel; ++blk) {
    const bool diag = blk == nsel;
    __syncthreads();
    if (tid < 32) {
      int key;
      if (diag) {
        key = tile_key0 + tid;
      } else {
        const int s = blk * 32 + tid;
        key = -1;
        if (s < kt) {
          const int j = S[s];
          key = ((unsigned)j < (unsigned)tile_key0) ? j : 0;   // trusted input, kept in bounds
        }
      }
      s_key[tid] = key;
    }
    __syncthreads();
    // K rows (row-major) and V rows transposed to [d][key]
    {
      constexpr int PARTS = D / 8;
      for (int x = tid; x < 32 * PARTS; x += NT) {
        const int r = x / PARTS, part = x % PARTS;
        const int key = s_key[r];
        *reinterpret_cast<u32x4*>(s_k + r * KROW + part * 16) =
            ldg16(kbase + (int64_t)(key < 0 ? 0 : key) * D + part * 8);
      }
      for (int x = tid; x < 16 * PARTS; x += NT) {
        const int kp = x / PARTS, part = x % PARTS;
        const int k0 = s_key[2 * kp], k1 = s_key[2 * kp + 1];
        const u32x4 v0 = ldg16(vbase + (int64_t)(k0 < 0 ? 0 : k0) * D + part * 8);
        const u32x4 v1 = ldg16(vbase + (int64_t)(k1 < 0 ? 0 : k1) * D + part * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = (v0[e] & 0xffffu) | (v1[e] << 16);          // dim 2e
          const uint32_t hi = (v0[e] >> 16) | (v1[e] & 0xffff0000u);      // dim 2e+1
          *reinterpret_cast<uint32_t*>(s_vt + (part * 8 + 2 * e) * VROW + 4 * kp) = lo;
          *reinterpret_cast<uint32_t*>(s_vt + (part * 8 + 2 * e + 1) * VROW + 4 * kp) = hi;
        }
      }
    }
    __syncthreads();
    f32x16 acc = {};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(s_k + n32 * KROW + (16 * c + 8 * hh) * 2);
      acc = mfma32(ka, qb[c], acc);             // S^T[key slot][query]
    }
    float x[16];
    float bm = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int slot = mrow(r, hh);
      const bool ok = diag ? (slot <= n32) : (s_key[slot] >= 0);
      x[r] = ok ? acc[r] * cs : kNegInf;
      bm = fmaxf(bm, x[r]);
    }
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    // lazy rescale: keep the running max unless a score exceeds it by 2^8
    const bool bump = (m_run == kNegInf) ? (bm != kNegInf) : (bm > m_run + 8.f);
    const float m_new = bump ? bm : m_run;
    const float alpha = bump ? ((m_run == kNegInf) ? 0.f : exp2_fast(m_run - m_new)) : 1.f;
    if (__any(bump)) {
      if (hh == 0) s_x[w][n32] = alpha;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      float ar[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ar[r] = s_x[w][mrow(r, hh)];
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dc][r] *= ar[r];
      __builtin_amdgcn_wave_barrier();
    }
    l_run *= alpha;
    m_run = m_new;
    float p[16];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = (x[r] == kNegInf) ? 0.f : exp2_fast(x[r] - m_run);
      ps += p[r];
    }
    l_run += ps;
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      u32x4 pa;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        pa[e] = (uint32_t)f32_to_bf16_rne(p[8 * c2 + 2 * e]) | ((uint32_t)f32_to_bf16_rne(p[8 * c2 + 2 * e + 1]) << 16);
#pragma unroll
      for (int dc = 0; dc < NDC; ++dc) {
        const char* vr = s_vt + (n32 + 32 * dc) * VROW;
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vr + (16 * c2 + 4 * hh) * 2);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vr + (16 * c2 + 8 + 4 * hh) * 2);
        const u32x4 vb = {lo[0], lo[1], hi[0], hi[1]};
        o[dc] = mfma32(pa, vb, o[dc]);
      }
    }
  }
  // normalise: row sums live with the query's lanes, output rows with registers
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  __syncthreads();
  if (hh == 0) s_x[w][n32] = 1.0f / l_tot;
  __syncthreads();
  float inv[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) inv[r] = s_x[w][mrow(r, hh)];
  uint16_t* ob = reinterpret_cast<uint16_t*>(a.o) + qoff * D;
#pragma unroll
  for (int dc = 0; dc < NDC; ++dc)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      ob[(int64_t)mrow(r, hh) * D + n32 + 32 * dc] = f32_to_bf16_rne(o[dc][r] * inv[r]);
}

// ------------------------------------------------------------------ host side

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

static int64_t pool_budget_floats() {
  const char* v = getenv("KAS_PREFILL_POOL_MB");
  int64_t mb = (v && atoll(v) > 0) ? atoll(v) : kPoolBudgetMBDefault;
  return mb * (1 << 20) / 4;
}

// Tiles [ta, tb) per pool/select launch so that the pooled rows fit the budget.
static int next_chunk_end(int ta, int T, int64_t units, int64_t budget) {
  int64_t used = 0;
  int tb = ta;
  while (tb < T) {
    const int64_t need = units * kTile * (int64_t)tb;
    if (tb > ta && used + need > budget) break;
    used += need;
    ++tb;
  }
  return tb;
}

static int64_t max_chunk_floats(int T, int64_t units, int64_t budget) {
  int64_t best = 0;
  for (int ta = 1; ta < T;) {
    const int tb = next_chunk_end(ta, T, units, budget);
    const int64_t f = units * kTile * ((int64_t)tb * (tb - 1) / 2 - (int64_t)ta * (ta - 1) / 2);
    best = f > best ? f : best;
    ta = tb;
  }
  return best;
}

struct PrefillPlan {
  size_t off_offsets, off_lse, off_pooled, total;
  int64_t pooled_floats;
};

static PrefillPlan plan(int B, int Hq, int Hkv, int64_t N, bool anchor) {
  PrefillPlan p{};
  const int T = (int)(N / kTile);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
  p.off_offsets = take((size_t)(T + 1) * sizeof(int32_t));
  if (anchor) {
    p.off_lse = take((size_t)B * Hq * N * sizeof(float));
    p.pooled_floats = max_chunk_floats(T, (int64_t)B * Hkv, pool_budget_floats());
    p.off_pooled = take((size_t)(p.pooled_floats > 0 ? p.pooled_floats : 1) * sizeof(float));
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
  PrefillPlan p = plan(B, Hq, Hkv, N, anchor);
  a.offsets = (int32_t*)(ws + p.off_offsets);
  if (anchor) {
    a.lse = (float*)(ws + p.off_lse);
    a.pooled = (float*)(ws + p.off_pooled);
    a.pooled_floats = (size_t)p.pooled_floats;
  }
}

#define KAS_LAUNCH_P(kernel, grid, block, stream, arg) \
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, arg)

#define KAS_DISPATCH_DG(KERNEL, grid, st, a)                                              \
  do {                                                                                    \
    if (a.D == 128) {                                                                     \
      switch (a.G) {                                                                      \
        case 1: KAS_LAUNCH_P((KERNEL<128, 1>), grid, dim3(64), st, a); break;             \
        case 2: KAS_LAUNCH_P((KERNEL<128, 2>), grid, dim3(128), st, a); break;            \
        case 4: KAS_LAUNCH_P((KERNEL<128, 4>), grid, dim3(256), st, a); break;            \
        case 8: KAS_LAUNCH_P((KERNEL<128, 8>), grid, dim3(512), st, a); break;            \
        default: return hipErrorInvalidValue;                                             \
      }                                                                                   \
    } else {                                                                              \
      switch (a.G) {                                                                      \
        case 1: KAS_LAUNCH_P((KERNEL<64, 1>), grid, dim3(64), st, a); break;              \
        case 2: KAS_LAUNCH_P((KERNEL<64, 2>), grid, dim3(128), st, a); break;             \
        case 4: KAS_LAUNCH_P((KERNEL<64, 4>), grid, dim3(256), st, a); break;             \
        case 8: KAS_LAUNCH_P((KERNEL<64, 8>), grid, dim3(512), st, a); break;             \
        default: return hipErrorInvalidValue;                                             \
      }                                                                                   \
    }                                                                                     \
  } while (0)

static hipError_t launch_offsets(PrefillArgs& a, LaunchCtx& ctx) {
  KAS_LAUNCH_P(pre_offsets_kernel, dim3(1), dim3(256), ctx.stream, a);
  return hipGetLastError();
}

static hipError_t launch_attn(PrefillArgs& a, LaunchCtx& ctx) {
  ctx.begin(K_PRE_ATTN);
  dim3 grid(a.T, a.Hkv, a.B);
  KAS_DISPATCH_DG(pre_attn_kernel, grid, ctx.stream, a);
  return ctx.end(K_PRE_ATTN);
}

hipError_t launch_prefill_anchor(PrefillArgs& a, LaunchCtx& ctx) {
  hipError_t e;
  if ((e = launch_offsets(a, ctx)) != hipSuccess) return e;
  ctx.begin(K_PRE_STATS);
  {
    dim3 grid(a.T, a.Hkv, a.B);
    KAS_DISPATCH_DG(pre_stats_kernel, grid, ctx.stream, a);
  }
  if ((e = ctx.end(K_PRE_STATS)) != hipSuccess) return e;
  const int64_t units = (int64_t)a.B * a.Hkv;
  const int64_t budget = pool_budget_floats();
  for (int ta = 1; ta < a.T;) {
    const int tb = next_chunk_end(ta, a.T, units, budget);
    a.t_begin = ta;
    a.t_end = tb;
    dim3 grid(tb - ta, a.Hkv, a.B);
    ctx.begin(K_PRE_POOL);
    KAS_DISPATCH_DG(pre_pool_kernel, grid, ctx.stream, a);
    if ((e = ctx.end(K_PRE_POOL)) != hipSuccess) return e;
    ctx.begin(K_PRE_SELECT);
    KAS_LAUNCH_P(pre_select_kernel, grid, dim3(256), ctx.stream, a);
    if ((e = ctx.end(K_PRE_SELECT)) != hipSuccess) return e;
    ta = tb;
  }
  return launch_attn(a, ctx);
}

hipError_t launch_prefill_reuse(PrefillArgs& a, LaunchCtx& ctx) {
  hipError_t e;
  if ((e = launch_offsets(a, ctx)) != hipSuccess) return e;
  return launch_attn(a, ctx);
}

}  // namespace kas
