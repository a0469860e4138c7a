// Optional clean-up of the expand layout for gfx950: zero the alignment
// padding rows of every expert segment, rows [offsets[e] + counts[e],
// offsets[e+1]), so a consumer that walks whole aligned segments (an expert
// GEMM over A-row tiles) reads zeros there instead of stale memory.
//
// The segments and their alignment follow the DeepEP overall-architecture
// page (EPHandle: expert_alignment, psum_num_recv_tokens_per_expert,
// num_expanded_tokens); the pages leave the content of padding rows open,
// and dispatch leaves them untouched.
//
// Design (MI355X): counts and offsets stay on the device, so the grid covers
// every possible padding row (E x (A-1) rows, one wave per 1 KiB slice of a
// row); a wave reads its expert's segment bounds once (wave-uniform) and
// exits if its row is not padding. Stores are non-temporal 16-byte zeros.
#include "ep_device.hpp"
#include "ep_launch.hpp"

namespace ep {
namespace {


// WIDE: launched over the whole chip (no workgroup cap), which selects the
// store policy: non-temporal at device scope like dispatch's rows
// (RowStore::kNtDevice); under a cap, non-temporal.
template <bool WIDE>
__global__ __launch_bounds__(kCappedThreads) void ep_zero_padding_rows(
    u32x4 *__restrict__ expand_x, int64_t row_chunks, float *__restrict__ expand_scales,
    int64_t scale_cols, float *__restrict__ expand_weights, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ offsets, int E, int A, int64_t capacity) {
  const int lane = lane_id();
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int64_t total = (int64_t)E * (A - 1) * slices;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  const int64_t stride = (int64_t)gridDim.x * wpb;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int64_t gw = (int64_t)blockIdx.x * wpb + wave_in_block; gw < total;
       gw += stride) {
    const int64_t er = gw / slices;
    const int64_t slice = gw - er * slices;
    const int e = (int)(er / (A - 1));
    const int r = (int)(er - (int64_t)e * (A - 1));
    const int64_t begin = (int64_t)__builtin_amdgcn_readfirstlane(offsets[e]) +
                          __builtin_amdgcn_readfirstlane(counts[e]);
    const int64_t end = __builtin_amdgcn_readfirstlane(offsets[e + 1]);
    const int64_t row = begin + r;
    if (row >= end || row >= capacity || row < 0) continue;
    const int64_t i = slice * kWave + lane;
    if (i < row_chunks)
      store_row<WIDE ? RowStore::kNtDevice : RowStore::kNt>(zero, expand_x + row * row_chunks,
                                                             (int)(row_chunks * 16), (int)(i * 16));
    if (slice == 0) {
      if (expand_scales != nullptr)
        for (int64_t j = lane; j < scale_cols; j += kWave)
          expand_scales[row * scale_cols + j] = 0.0f;
      if (expand_weights != nullptr && lane == 0) expand_weights[row] = 0.0f;
    }
  }
}

}  // namespace

int launch_zero_padding(const ZeroPaddingArgs &a) {
  if (a.A <= 1) return 0;  // no padding rows exist
  const int64_t row_chunks = a.row_bytes / 16;
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int cap = stream_workgroup_limit(a.stream);
  const WaveGrid g = wave_grid((int64_t)a.E * (a.A - 1) * slices, cap, 1 << 22);
  if (cap > 0)
    ep_zero_padding_rows<false><<<g.blocks, g.threads, 0, a.stream>>>(
        (u32x4 *)a.expand_x, row_chunks, a.expand_scales, a.scale_cols, a.expand_weights, a.counts,
        a.offsets, a.E, a.A, a.capacity);
  else
    ep_zero_padding_rows<true><<<g.blocks, g.threads, 0, a.stream>>>(
        (u32x4 *)a.expand_x, row_chunks, a.expand_scales, a.scale_cols, a.expand_weights, a.counts,
        a.offsets, a.E, a.A, a.capacity);
  return launch_status();
}

}  // namespace ep
