// Device helpers shared by the gfx950 kernels: element loads and conversion,
// wavefront reductions, MFMA wrappers and the base-2 exponential.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kas {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// log2(e): logits are kept in base-2 units so that softmax uses v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// bf16 bit pattern in the low / high half of a dword -> fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// acc + (lo + hi) of a packed bf16 pair, in one dot product with (1, 1)
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4v __attribute__((ext_vector_type(4)));

// The two 16-bit element types of the matrix paths (bf16, fp16): their MFMA
// instructions (operands as raw dwords, 8 or 4 elements per lane), the
// round-to-nearest-even packing of two fp32 values, the exact fp32 sum of a
// packed pair (a dot product with (1, 1)), the rounding store, and the
// largest half-row probability sum the lazy softmax lets grow before it
// rescales (bf16 shares fp32's exponent range; fp16 ends at 65504).
template <typename E>
struct Ew;

template <>
struct Ew<__bf16> {
  static constexpr float kBigP = 0x1p64f;
  __device__ static __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4v, a), __builtin_bit_cast(i16x4v, b),
                                                     c, 0, 0, 0);
  }
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
  __device__ static __forceinline__ float add2(uint32_t pair, float acc) { return add_bf16x2(pair, acc); }
  __device__ static __forceinline__ uint16_t bits(float f) { return f32_to_bf16_rne(f); }
};

template <>
struct Ew<_Float16> {
  static constexpr float kBigP = 0x1p14f;
  __device__ static __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  c, 0, 0, 0);
  }
  __device__ static __forceinline__ f32x4 mfma16k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b),
                                                 c, 0, 0, 0);
  }
  // v_cvt_pk_f16_f32 (round to nearest even)
  __device__ static __forceinline__ uint32_t pack2(float lo, float hi) {
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
  __device__ static __forceinline__ float add2(uint32_t pair, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
  }
  __device__ static __forceinline__ uint16_t bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
};

// ---------------------------------------------------------------- DPP
// Reductions inside each row of 16 lanes; afterwards every lane of the row
// holds the row's result.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuad1032 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuad2301 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<kDppQuad1032>(x));
  x = fmaxf(x, dpp_f<kDppQuad2301>(x));
  x = fmaxf(x, dpp_f<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppRowMirror>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<kDppQuad1032>(x);
  x += dpp_f<kDppQuad2301>(x);
  x += dpp_f<kDppRowHalfMirror>(x);
  x += dpp_f<kDppRowMirror>(x);
  return x;
}

// Combine each lane's value with that of lane l ^ 32 without an LDS round
// trip. v_permlane32_swap exchanges the upper half-wave of its first operand
// with the lower half-wave of its second; fed x twice, its two results hold
// x[l] and x[l ^ 32] (in an order that differs between the halves), so a
// symmetric combination of them gives the same value in lanes l and l ^ 32.
__device__ __forceinline__ float xor32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Maximum of the 16 accumulator values of a 32x32 MFMA tile held by a lane,
// as a depth-three tree of three-input maxima.
template <typename V>
__device__ __forceinline__ float max16(const V& v) {
  const float t0 = fmaxf(fmaxf(v[0], v[1]), v[2]), t1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
  const float t2 = fmaxf(fmaxf(v[6], v[7]), v[8]), t3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
  const float t4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(t0, t1), t2), fmaxf(fmaxf(t3, t4), v[15]));
}

// Full 64-lane reductions through cross-lane permutes.
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// ---------------------------------------------------------------- loads
// 16-byte global load of 8 bf16 (as raw dwords).
__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// 16 bytes with the non-temporal hint (the line is not kept in the caches)
__device__ __forceinline__ u32x4 ldg16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ldg8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Load EPL consecutive elements of T at p and widen to fp32.
template <typename T, int EPL>
struct RowFrag;

template <>
struct RowFrag<__bf16, 8> {
  u32x4 w;
  __device__ __forceinline__ void load(const __bf16* p) { w = ldg16(p); }
  __device__ __forceinline__ void widen(float* f) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16lo(w[i]); f[2 * i + 1] = bf16hi(w[i]); }
  }
};
template <>
struct RowFrag<__bf16, 4> {
  u32x2 w;
  __device__ __forceinline__ void load(const __bf16* p) { w = ldg8(p); }
  __device__ __forceinline__ void widen(float* f) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) { f[2 * i] = bf16lo(w[i]); f[2 * i + 1] = bf16hi(w[i]); }
  }
};
template <>
struct RowFrag<float, 4> {
  u32x4 w;
  __device__ __forceinline__ void load(const float* p) { w = ldg16(p); }
  __device__ __forceinline__ void widen(float* f) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
};
template <>
struct RowFrag<float, 8> {
  u32x4 w0, w1;
  __device__ __forceinline__ void load(const float* p) { w0 = ldg16(p); w1 = ldg16(p + 4); }
  __device__ __forceinline__ void widen(float* f) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = __uint_as_float(w0[i]); f[4 + i] = __uint_as_float(w1[i]); }
  }
};

// ---------------------------------------------------------------- MFMA QK
// Q.K^T for one block of 16 keys against up to 16 query heads on a 16x16
// MFMA tile: A = Q (row m = head = lane % 16), B = K^T (column n = key =
// lane % 16), contraction over head_dim. Output lane l, reg r holds
// S[head = 4*(l/16) + r][key = l % 16]. Both operands use the same split of
// head_dim across lanes, so the hardware's k-order inside an instruction does
// not matter.
template <typename T, int D>
struct QKMfma;

// 16-bit elements (bf16, fp16): v_mfma_f32_16x16x32_{bf16,f16}; instruction
// c covers dims [32c, 32c+32), lane quarter q = l/16 supplies dims 32c + 8q .. +8.
template <typename E, int D>
struct QKMfma16 {
  static constexpr int NI = D / 32;
  u32x4 kf[NI];
  __device__ __forceinline__ static int dim_of(int c, int q) { return 32 * c + 8 * q; }
  __device__ __forceinline__ void load_k(const E* row, int q) {
#pragma unroll
    for (int c = 0; c < NI; ++c) kf[c] = ldg16(row + dim_of(c, q));
  }
  // the same with non-temporal loads (rows read once per call)
  __device__ __forceinline__ void load_k_nt(const E* row, int q) {
#pragma unroll
    for (int c = 0; c < NI; ++c) kf[c] = ldg16_nt(row + dim_of(c, q));
  }
  struct QFrag { u32x4 a[NI]; };
  __device__ __forceinline__ static void load_q(QFrag& f, const E* qrow, bool valid, int q) {
#pragma unroll
    for (int c = 0; c < NI; ++c) f.a[c] = valid ? ldg16(qrow + dim_of(c, q)) : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ f32x4 run(const QFrag& f) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NI; ++c) acc = Ew<E>::mfma16k32(f.a[c], kf[c], acc);
    return acc;
  }
};
template <int D>
struct QKMfma<__bf16, D> : QKMfma16<__bf16, D> {};
template <int D>
struct QKMfma<_Float16, D> : QKMfma16<_Float16, D> {};

// fp32: v_mfma_f32_16x16x4_f32; lane quarter q owns dims [q*D/4, (q+1)*D/4)
// (contiguous, loaded 16 B at a time) and instruction c uses its c-th dim.
template <int D>
struct QKMfma<float, D> {
  static constexpr int NI = D / 4;
  static constexpr int NV = NI / 4;   // 16-byte vectors per lane
  u32x4 kf[NV];
  __device__ __forceinline__ void load_k(const float* row, int q) {
#pragma unroll
    for (int c = 0; c < NV; ++c) kf[c] = ldg16(row + q * NI + 4 * c);
  }
  struct QFrag { u32x4 a[NV]; };
  __device__ __forceinline__ static void load_q(QFrag& f, const float* qrow, bool valid, int q) {
#pragma unroll
    for (int c = 0; c < NV; ++c) f.a[c] = valid ? ldg16(qrow + q * NI + 4 * c) : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ f32x4 run(const QFrag& f) const {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NV; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.a[c][e]), __uint_as_float(kf[c][e]),
                                                   acc, 0, 0, 0);
    return acc;
  }
};

}  // namespace kas
