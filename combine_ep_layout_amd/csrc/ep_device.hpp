// Device helpers shared by the gfx950 kernels of this library (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// 64-bit ballot over the wavefront.
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes strictly below the calling lane.
__device__ __forceinline__ int count_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Value of `v` held by lane `src` (src must be wave-uniform).
__device__ __forceinline__ int read_lane(int v, int src) { return __builtin_amdgcn_readlane(v, src); }
__device__ __forceinline__ float read_lane(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Exclusive prefix sum of one value per thread over a block of NT threads.
// `s_tmp` holds NT/64 ints of LDS. Returns the exclusive prefix; `total`
// receives the block-wide sum. Contains barriers: call from every thread.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_tmp, int &total) {
  constexpr int NW = NT / kWave;
  static_assert(NW <= kWave, "block too large for a two-level scan");
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int inc = wave_inclusive_scan(v);
  if (lane == kWave - 1) s_tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    int s = lane < NW ? s_tmp[lane] : 0;
    s = wave_inclusive_scan(s);
    if (lane < NW) s_tmp[lane] = s;
  }
  __syncthreads();
  const int before = w ? s_tmp[w - 1] : 0;
  total = s_tmp[NW - 1];
  __syncthreads();
  return before + inc - v;
}

}  // namespace ep
