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

// Inclusive scan of a 32-bit int over a wave64 with DPP lane moves (no LDS
// traffic): a Hillis-Steele scan inside each row of 16 lanes (row_shr 1, 2,
// 4, 8), then row 1 adds lane 15 and row 3 lane 47 (row_bcast:15), and rows
// 2 and 3 add lane 31 (row_bcast:31). Lanes a move has no source for get 0.
__device__ __forceinline__ int32_t wave_incl_scan_dpp(int32_t x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Inclusive running maximum of a non-negative int over a wave64, with the
// same DPP lane moves as wave_incl_scan_dpp (0 is the identity).
__device__ __forceinline__ int32_t wave_incl_max_dpp(int32_t x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true));  // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true));  // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true));  // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true));  // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return x;
}

// A double moved between lanes by one DPP control (each 32-bit half moved
// alike); lanes the move has no source for, or rows outside ROW_MASK, get 0.
template <int CTRL, int ROW_MASK, bool BOUND_CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROW_MASK,
                                                            0xf, BOUND_CTRL);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL,
                                                            ROW_MASK, 0xf, BOUND_CTRL);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum of a double over a wave64, in lane 63 (the other lanes hold partial
// sums): the lane moves of wave_incl_scan_dpp, no LDS traffic. Every lane
// must be active.
__device__ __forceinline__ double wave_total_f64(double x) {
  x += dpp_f64<0x111, 0xf, true>(x);   // row_shr:1
  x += dpp_f64<0x112, 0xf, true>(x);   // row_shr:2
  x += dpp_f64<0x114, 0xf, true>(x);   // row_shr:4
  x += dpp_f64<0x118, 0xf, true>(x);   // row_shr:8
  x += dpp_f64<0x142, 0xa, false>(x);  // row_bcast:15
  x += dpp_f64<0x143, 0xc, false>(x);  // row_bcast:31
  return x;
}

// Block-wide inclusive scan of a 32-bit int with one barrier. `ws` is NT/64
// ints of LDS that the caller must not reuse before another barrier: two
// calls need a barrier between them (the second would overwrite `ws` while
// slower waves of the first still read it).
template <int NT>
__device__ __forceinline__ int32_t block_incl_scan_1b(int32_t v, int32_t *ws, int32_t *total) {
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int32_t x = wave_incl_scan_dpp(v);
  asm volatile("" : "+v"(x));  // keep the scan, not its partial terms, across the barrier
  if (lane == 63) ws[w] = x;
  __syncthreads();
  int32_t off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int32_t s = ws[i];
    if (i < w) off += s;
    tot += s;
  }
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
