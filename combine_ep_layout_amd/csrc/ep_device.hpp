// Device helpers shared by the gfx950 kernels of this library (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Cache policy of a row store.
//   kNt:       non-temporal (global_store ... nt).
//   kNtDevice: non-temporal at device scope (gfx950 `nt sc1`): the line is
//              written towards memory without being kept in this XCD's L2.
//   kDevice:   device scope, kept (`sc1` alone).
// Measured on MI355X with the whole chip storing: dispatch's expand rows
// (470 MB at prefill, more than the 256 MB last-level cache) are fastest with
// kNtDevice (87.5 against 91.7 us with kNt, about 160 us with kDevice or plain
// stores); combine's output rows (59 MB, which fit that cache) are fastest
// with kDevice (86.9 against 91.6 us with kNt, 90.3 with kNtDevice, 93.4
// plain). Under a workgroup cap device scope is much slower (fan-out dispatch
// 183 against 115 us on 64 workgroups) or no better, so capped launches use
// kNt.
enum class RowStore { kNt, kNtDevice, kDevice };

// Stores 16 bytes at byte offset `off` of a row of `row_bytes` bytes that
// starts at `row` (wave-uniform) with policy P. The two device-scope policies
// go through a buffer resource built from the row pointer, so the offset
// stays small however large the buffer is and a lane past the row's end
// writes nothing.
template <RowStore P>
__device__ __forceinline__ void store_row(const u32x4 &v, void *row, int row_bytes, int off) {
  if constexpr (P == RowStore::kNt) {
    __builtin_nontemporal_store(v, (u32x4 *)((char *)row + off));
  } else {
    constexpr int kNt = 2, kSc1 = 16;            // cache-policy bits of a buffer store
    constexpr int kRawBufferFlags = 0x00020000;  // buffer descriptor word 3 for gfx9-family parts
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(row, (short)0, row_bytes, kRawBufferFlags);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, off, 0,
                                           P == RowStore::kNtDevice ? kNt | kSc1 : kSc1);
  }
}

// Waits until every vector memory operation this wave has issued is done
// (s_waitcnt with vmcnt 0 and the expcnt and lgkmcnt fields at their maxima,
// which leaves those two counters free; gfx9-family immediate layout:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits 15:14). A
// kernel that loads once and then stores under several wave-uniform branches
// calls it between the two: the compiler cannot count outstanding operations
// across those branches and otherwise waits for the previous store before
// each store.
__device__ __forceinline__ void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// 64-bit ballot over the wavefront.
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes strictly below the calling lane.
__device__ __forceinline__ int count_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Value of `v` held by lane `src` (src must be wave-uniform).
__device__ __forceinline__ int read_lane(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}
__device__ __forceinline__ float read_lane(float v, int src) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// Inclusive prefix sum within each row of 16 lanes, in registers: DPP row
// shifts by 1, 2, 4 and 8 lanes (a lane whose source falls outside its row
// adds 0).
__device__ __forceinline__ int row_inclusive_scan(int x) {
  constexpr int kRowShr = 0x110;  // DPP control row_shr:n is kRowShr + n
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 2, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 4, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 8, 0xF, 0xF, false);
  return x;
}

// Inclusive prefix sum over the 64 lanes of a wavefront: row scans, then
// each lane adds the totals of the rows below its own (last lane of each
// row, read with readlane). No LDS traffic, unlike lane shuffles.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x = row_inclusive_scan(x);
  const int lane = lane_id();
  const int r0 = __builtin_amdgcn_readlane(x, 15);
  const int r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// Sum over the 64 lanes of a wavefront (the same value in every lane).
__device__ __forceinline__ int wave_sum(int x) {
  x = row_inclusive_scan(x);
  return __builtin_amdgcn_readlane(x, 15) + __builtin_amdgcn_readlane(x, 31) +
         __builtin_amdgcn_readlane(x, 47) + __builtin_amdgcn_readlane(x, 63);
}

}  // namespace ep
