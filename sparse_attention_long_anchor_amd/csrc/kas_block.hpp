// Workgroup-level helpers (256-thread workgroups unless stated): reductions,
// exclusive scans and the radix-select bin search.
#pragma once
#include "kas_device.hpp"

namespace kas {

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float block_max_256(float x, float* s_tmp) {
  x = wave_max(x);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_tmp[wave] = x;
  __syncthreads();
  return fmaxf(fmaxf(s_tmp[0], s_tmp[1]), fmaxf(s_tmp[2], s_tmp[3]));
}
__device__ __forceinline__ float block_sum_256(float x, float* s_tmp) {
  x = wave_sum(x);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_tmp[wave] = x;
  __syncthreads();
  return (s_tmp[0] + s_tmp[1]) + (s_tmp[2] + s_tmp[3]);
}
// Exclusive prefix over the 256 threads (thread order).
__device__ __forceinline__ uint32_t block_excl_scan_256(uint32_t x, uint32_t* s_tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = wave_incl_scan_u32(x);
  __syncthreads();
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wave; ++w) before += s_tmp[w];
  if (total) *total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  return before + inc - x;
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bin holding the krem-th largest element (1-based) and the count above it.
__device__ __forceinline__ void block_find_bin(const uint32_t* hist, int nbins, uint32_t krem, uint32_t* s_tmp,
                               int* s_res, int& bin, uint32_t& above) {
  const int tid = threadIdx.x;
  const int per = nbins / 256;
  const int hi = nbins - tid * per;
  if (tid == 0) { s_res[0] = 0; s_res[1] = 0; }
  uint32_t local = 0;
  for (int x = hi - per; x < hi; ++x) local += hist[x];
  uint32_t excl = block_excl_scan_256(local, s_tmp, nullptr);
  if (excl < krem && excl + local >= krem) {
    uint32_t acc = excl;
    for (int x = hi - 1; x >= hi - per; --x) {
      uint32_t c = hist[x];
      if (acc + c >= krem) { s_res[0] = x; s_res[1] = (int)acc; break; }
      acc += c;
    }
  }
  __syncthreads();
  bin = s_res[0];
  above = (uint32_t)s_res[1];
  __syncthreads();
}


// ---------------------------------------------------------------- NT-thread variants

template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* s_tmp, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t inc = wave_incl_scan_u32(x);
  __syncthreads();
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t v = s_tmp[w];
    before += (w < wave) ? v : 0u;
    all += v;
  }
  if (total) *total = all;
  return before + inc - x;
}

// Bin holding the krem-th largest element (1-based) of an nbins histogram
// (nbins a multiple of NT) and the count of elements in higher bins.
template <int NT>
__device__ __forceinline__ void block_find_bin_nt(const uint32_t* hist, int nbins, uint32_t krem, uint32_t* s_tmp,
                                                  int* s_res, int& bin, uint32_t& above) {
  const int tid = threadIdx.x;
  const int per = nbins / NT;
  const int hi = nbins - tid * per;
  if (tid == 0) { s_res[0] = 0; s_res[1] = 0; }
  uint32_t local = 0;
  for (int x = hi - per; x < hi; ++x) local += hist[x];
  const uint32_t excl = block_excl_scan<NT>(local, s_tmp, nullptr);
  if (excl < krem && excl + local >= krem) {
    uint32_t acc = excl;
    for (int x = hi - 1; x >= hi - per; --x) {
      const uint32_t c = hist[x];
      if (acc + c >= krem) { s_res[0] = x; s_res[1] = (int)acc; break; }
      acc += c;
    }
  }
  __syncthreads();
  bin = s_res[0];
  above = (uint32_t)s_res[1];
  __syncthreads();
}

}  // namespace kas
