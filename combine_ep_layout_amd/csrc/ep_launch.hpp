// Host-side interface between the C ABI (ep_capi.cpp) and the kernel
// launchers (ep_layout.hip, ep_dispatch.hip, ep_combine.hip). Arguments are
// validated by the C ABI before any launcher is called.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "ep_mi355x.h"

// The compiled shape set. Shapes are template constants of the kernels, so
// loops over a row and over k unroll completely; anything outside these
// lists is rejected by the capability gate in the C ABI.
#define EP_FOR_EACH_TOPK(X) X(1) X(2) X(4) X(6) X(8)
#define EP_FOR_EACH_HIDDEN_BF16(X) X(256) X(512) X(1024) X(2048) X(4096) X(7168)
#define EP_FOR_EACH_HIDDEN_FP32(X) X(256) X(512) X(1024) X(2048) X(4096) X(7168)
#define EP_FOR_EACH_HIDDEN_FP8(X) X(512) X(1024) X(2048) X(4096) X(7168)
// fp4x2: hidden counts bytes (two e2m1 values per byte); 3584 bytes = 7168 values.
#define EP_FOR_EACH_HIDDEN_FP4X2(X) X(256) X(512) X(1024) X(2048) X(3584)

namespace ep {

struct LayoutArgs {
  const int32_t *topk_idx;
  int T, K, E, A;
  int32_t *counts, *offsets, *dst_slot, *meta, *num_recv;
  void *workspace;
  int32_t *plan;  // [T*K] (entry, slot) pairs, or NULL
  hipStream_t stream;
  const void *prefetch = nullptr;  // memory to read ahead into the last-level cache, or NULL
  int64_t prefetch_bytes = 0;
};

struct DispatchArgs {
  const void *x;
  const float *x_scales;
  const float *topk_weights;
  const int32_t *dst_slot;
  int T, H, K, dtype;
  int64_t capacity;
  void *expand_x;
  float *expand_scales;
  float *expand_weights;
  const int32_t *plan;  // [T*K] (entry, slot) pairs from ep_layout, or NULL
  hipStream_t stream;
};

struct CombineArgs {
  const void *y;
  const float *topk_weights;
  const void *bias;
  const int32_t *dst_slot;
  int T, H, K, dtype;
  int64_t capacity;
  void *out;
  hipStream_t stream;
};

struct ZeroPaddingArgs {
  void *expand_x;
  int64_t row_bytes;
  float *expand_scales;
  int64_t scale_cols;
  float *expand_weights;
  const int32_t *counts, *offsets;
  int E, A;
  int64_t capacity;
  hipStream_t stream;
};

struct CompactDispatchArgs {
  const void *x;
  int64_t row_bytes;
  const float *x_scales;
  int64_t scale_cols;
  const int32_t *topk_idx;
  const float *topk_weights;
  const int32_t *dst_slot, *meta, *num_recv;
  int T, K;
  void *recv_x;
  float *recv_scales;
  int32_t *recv_topk_idx;
  float *recv_topk_weights;
  hipStream_t stream;
};

struct CompactCombineArgs {
  const void *y;
  int64_t row_bytes;
  const void *bias;
  const int32_t *dst_slot, *meta, *num_recv;
  int T, K;
  void *out;
  hipStream_t stream;
  bool fp32 = false;  // binary32 rows (else bf16)
};

// Launch geometry. By default a grid covers every unit of work with
// 256-thread workgroups, so the hardware spreads it over all compute units.
// A stream may carry a workgroup cap (ep_set_workgroup_limit): every kernel
// launched on it then uses at most that many workgroups, each large enough to
// keep one compute unit's memory pipeline busy (1024 threads for kernels
// whose waves move 1 KiB at a time, fewer for kernels with more loads in
// flight per wave), and its waves loop over the work, leaving the other
// compute units free for work on other streams.
constexpr int kDefaultThreads = 256;
constexpr int kCappedThreads = 1024;

// Division of n < 2^31 by a divisor d (1 <= d < 2^31) fixed per launch, by
// multiplication: q = (n * m) >> s with s = 31 + ceil(log2 d) and
// m = floor(2^s / d) + 1 (below 2^32). m exceeds 2^s / d by at most 1, so
// n * m / 2^s exceeds n / d by less than n / 2^s < 2^-ceil(log2 d) <= 1 / d,
// which never reaches the next multiple of 1 / d above n / d: the floor is
// exact. Costs a 32 x 32 -> 64-bit multiply and a shift instead of a
// division sequence.
struct FastDiv {
  uint32_t m, s;
};
inline FastDiv fast_div(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  return {(uint32_t)((uint64_t(1) << (31 + l)) / d + 1), 31 + l};
}
__device__ __forceinline__ uint32_t fast_div_apply(uint32_t n, FastDiv f) {
  return (uint32_t)(((uint64_t)n * f.m) >> f.s);
}

// Units (one wave each) per launch of a kernel whose uncapped waves move one
// unit and exit: 2^24 - 16 workgroups of four waves (a multiple of 8, within
// the grid limit of 2^32 threads). Larger inputs take further launches, each
// from a unit offset. A test build sets EP_MAX_LAUNCH_UNITS to a few thousand
// so that those paths run on small inputs.
#ifndef EP_MAX_LAUNCH_UNITS
#define EP_MAX_LAUNCH_UNITS ((int64_t(1) << 26) - 64)
#endif
constexpr int64_t kMaxLaunchUnits = EP_MAX_LAUNCH_UNITS;

// The cap registered for this stream handle, or 0 for none.
int stream_workgroup_limit(hipStream_t stream);

struct WaveGrid {
  unsigned blocks;
  int threads;
};

// Grid for `waves` independent one-wave units (at least one workgroup) under
// the workgroup cap `cap` (0: none; read once per launch with
// stream_workgroup_limit, so a concurrent change cannot split one launch's
// decisions). max_blocks bounds the uncapped grid (larger inputs loop);
// round_to, if above 1, rounds the uncapped block count up to a multiple of
// it; capped_threads is the workgroup size under a cap (the kernel's launch
// bound).
inline WaveGrid wave_grid(int64_t waves, int cap, int64_t max_blocks, int round_to = 1,
                          int capped_threads = kCappedThreads) {
  const int threads = cap > 0 ? capped_threads : kDefaultThreads;
  const int wpb = threads / 64;
  int64_t blocks = (waves + wpb - 1) / wpb;
  if (blocks > max_blocks) blocks = max_blocks;
  if (cap > 0) {
    if (blocks > cap) blocks = cap;
  } else if (round_to > 1) {
    blocks = (blocks + round_to - 1) / round_to * round_to;
  }
  return {(unsigned)(blocks > 0 ? blocks : 1), threads};
}

// HIP error of the last failed launch on this thread (set by launch_status).
hipError_t &last_hip_error();

// Checks the launch just enqueued: 0, or -1 with last_hip_error() set.
inline int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return 0;
  last_hip_error() = e;
  return -1;
}

// Each returns 0 on success, -1 if the HIP runtime reported an error on
// launch, -2 if the shape has no compiled kernel.
int launch_layout(const LayoutArgs &a);
size_t layout_workspace(int T, int K, int E);
// Device address of `device`'s copy of the library's fixed layout scratch
// (EP_LAYOUT_SCRATCH_BYTES), resolved on the first call for that device; the
// device must be current. Used by ep_layout_noalloc in place of a workspace.
hipError_t layout_scratch(int device, void **ptr);
int launch_dispatch(const DispatchArgs &a);
// Layout and dispatch in one launch when T*K fits one layout tile; -3 when it
// does not (the caller then launches them separately). Row and scale-row
// widths in 16-byte chunks.
int launch_layout_dispatch(const LayoutArgs &l, const DispatchArgs &d, int row_chunks,
                           int scale_chunks);
int launch_combine(const CombineArgs &a);
int launch_zero_padding(const ZeroPaddingArgs &a);
int launch_dispatch_compact(const CompactDispatchArgs &a);
// Layout and non-expand dispatch in one launch when T*K fits one layout tile;
// -3 when it does not. The dispatch arguments' dst_slot, meta and num_recv
// are the layout's outputs.
int launch_layout_dispatch_compact(const LayoutArgs &l, const CompactDispatchArgs &d);
int launch_combine_compact(const CompactCombineArgs &a);

bool has_layout(int K);
bool has_dispatch(int H, int K, int dtype);
bool has_combine(int H, int K, int dtype);

}  // namespace ep
