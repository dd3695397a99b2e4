// sps_device.h -- small wave64 / workgroup helpers shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sps {

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// inclusive scan over a wave64
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide inclusive scan for NT threads; `ws` is NT/64 elements of LDS.
// Returns the inclusive prefix; *total receives the block sum.
template <int NT, typename T>
__device__ __forceinline__ T block_incl_scan(T v, T *ws, T *total) {
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  T x = wave_incl_scan(v);
  if (lane == 63) ws[w] = x;
  __syncthreads();
  T off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    T s = ws[i];
    if (i < w) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return x + off;
}

// position of d in the ascending list heavy[0..m), or -1
__device__ __forceinline__ int heavy_slot(const int32_t *__restrict__ heavy, int m, int32_t d) {
  int lo = 0, hi = m;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (heavy[mid] < d) lo = mid + 1;
    else hi = mid;
  }
  return (lo < m && heavy[lo] == d) ? lo : -1;
}

}  // namespace sps
