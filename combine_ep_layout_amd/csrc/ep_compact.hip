// Non-expand dispatch and combine for gfx950: one row per received token.
//
// Follows the DeepEP overall-architecture page: EPHandle do_expand = false
// and the dispatch data-flow figure, whose copy epilogue writes recv_x,
// recv_topk_idx and recv_topk_weights; the combine reduce epilogue adds a
// bias. In a world of one every token with an unmasked entry is received
// exactly once, in ascending token order (recv_src_metadata), and the expert
// side returns one row per received token with its experts already reduced,
// so combine puts rows back in token order and adds the bias.
//
// Design (MI355X): both are row moves. One wave64 per (row, 1 KiB slice),
// 16-byte loads and non-temporal 16-byte stores; the number of received rows
// stays on the device, so the grid covers T rows and waves past num_recv
// exit. Shapes are run-time values here: there is no per-element arithmetic
// to unroll beyond the bias add. Uncapped, each wave moves one unit and exits
// (no grid-stride loop, so the compiler loads each kernel argument where it
// is first used): combine 17.4 against 19.0 us at prefill, 5.0 against 5.8 at
// mori_default, 36.4 against 38.0 at fp8_hot8; dispatch unchanged at prefill,
// 5.2 against 5.5 at mori_default (MI355X). Uncapped waves also find their
// row with 32-bit indices and a multiply-shift division by the slice count
// (FastDiv) instead of a 64-bit division sequence: combine 16.6 against 17.3
// us at prefill, 4.7 against 5.1 at mori_default; dispatch 4.9 against 5.3 at
// mori_default. Under a cap the waves loop.
#include "ep_device.hpp"
#include "ep_launch.hpp"

namespace ep {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// WIDE: launched over the whole chip (no workgroup cap), which selects the
// store policy: the receive rows and combine's output rows (one row per
// token, 59 MB at prefill) are stored at device scope and kept
// (RowStore::kDevice), unless they are larger than the last-level cache can
// keep beside the other traffic (stream_out: more than 128 MiB), when they
// are stored non-temporally at device scope (RowStore::kNtDevice; 32K tokens,
// 470 MB of rows: dispatch 152.2 against 157.8 us, step 308.7 against 322.5;
// at 117 MB, fp8_hot8, the kept rows are faster: combine 36.4 against 38.0).
// Under a cap, non-temporally.
template <bool WIDE>
__device__ __forceinline__ void store_out_row(const u32x4 &v, void *row, int row_bytes, int off,
                                              int stream_out) {
  if constexpr (!WIDE) {
    store_row<RowStore::kNt>(v, row, row_bytes, off);
  } else if (stream_out) {
    store_row<RowStore::kNtDevice>(v, row, row_bytes, off);
  } else {
    store_row<RowStore::kDevice>(v, row, row_bytes, off);
  }
}

template <bool WIDE>
__global__ __launch_bounds__(kCappedThreads) void ep_dispatch_compact_rows(
    const u32x4 *__restrict__ x, int64_t row_chunks, const float *__restrict__ x_scales,
    int64_t scale_cols, const int32_t *__restrict__ topk_idx,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ dst_slot,
    const int32_t *__restrict__ meta, const int32_t *__restrict__ num_recv, int T, int K,
    u32x4 *__restrict__ recv_x, float *__restrict__ recv_scales,
    int32_t *__restrict__ recv_topk_idx, float *__restrict__ recv_topk_weights,
    FastDiv by_slices, int stream_out) {
  const int lane = lane_id();
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int64_t total = (int64_t)T * slices;
  const int n = __builtin_amdgcn_readfirstlane(*num_recv);
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  auto move = [&](int64_t i, int64_t slice) {  // receive row i, slice
    if (i >= n) return;
    const int64_t t = __builtin_amdgcn_readfirstlane(meta[i * (K + 2)]);
    if (t < 0 || t >= T) return;
    const int64_t c = slice * kWave + lane;
    if (c < row_chunks)
      store_out_row<WIDE>(x[t * row_chunks + c], recv_x + i * row_chunks,
                          (int)(row_chunks * 16), (int)(c * 16), stream_out);
    if (slice == 0) {
      if (recv_scales != nullptr)
        for (int64_t j = lane; j < scale_cols; j += kWave)
          recv_scales[i * scale_cols + j] = x_scales[t * scale_cols + j];
      for (int k = lane; k < K; k += kWave) {
        const int64_t tk = t * K + k;
        recv_topk_idx[i * K + k] = dst_slot[tk] >= 0 ? topk_idx[tk] : -1;
        if (recv_topk_weights != nullptr) recv_topk_weights[i * K + k] = topk_weights[tk];
      }
    }
  };
  if constexpr (WIDE) {  // one unit per wave, all of them in this launch (total < 2^26)
    const uint32_t w = blockIdx.x * (uint32_t)wpb + wave_in_block;
    if (w >= (uint32_t)total) return;
    const uint32_t i = fast_div_apply(w, by_slices);
    move(i, w - i * (uint32_t)slices);
  } else {
    const int64_t stride = (int64_t)gridDim.x * wpb;
    for (int64_t gw = (int64_t)blockIdx.x * wpb + wave_in_block; gw < total; gw += stride) {
      const int64_t i = gw / slices;
      move(i, gw - i * slices);
    }
  }
}

// out[t] chunk c = v (+ bias[t] chunk c), one binary32 add per value; bf16
// rows (FP32 false) are widened exactly and the sum rounded back to bf16
// (round to nearest even), binary32 rows keep the sum as it is.
template <bool WIDE, bool FP32>
__device__ __forceinline__ void put_row_chunk(u32x4 v, const u32x4 *__restrict__ bias, int64_t t,
                                              int64_t row_chunks, int64_t c,
                                              u32x4 *__restrict__ out, int stream_out) {
#pragma clang fp contract(off)
  if (bias != nullptr) {
    const u32x4 b = bias[t * row_chunks + c];
    u32x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FP32) {
        r[j] = __float_as_uint(__uint_as_float(v[j]) + __uint_as_float(b[j]));
      } else {
        const float lo = __uint_as_float(v[j] << 16) + __uint_as_float(b[j] << 16);
        const float hi =
            __uint_as_float(v[j] & 0xffff0000u) + __uint_as_float(b[j] & 0xffff0000u);
        r[j] = pack_bf16x2(lo, hi);
      }
    }
    v = r;
  }
  store_out_row<WIDE>(v, out + t * row_chunks, (int)(row_chunks * 16), (int)(c * 16),
                      stream_out);
}

// Waves [0, T*slices): (receive row, slice) back to its token. Waves
// [T*slices, T*slices + T): one per token; a token with no unmasked entry
// (none of its K slots valid) gets +0 (+ bias) over its whole row, the
// others exit after one K-wide read.
template <bool WIDE, bool FP32>
__global__ __launch_bounds__(kCappedThreads) void ep_combine_compact_rows(
    const u32x4 *__restrict__ y, int64_t row_chunks, const u32x4 *__restrict__ bias,
    const int32_t *__restrict__ dst_slot, const int32_t *__restrict__ meta,
    const int32_t *__restrict__ num_recv, int T, int K, u32x4 *__restrict__ out,
    FastDiv by_slices, int stream_out) {
  const int lane = lane_id();
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int64_t half = (int64_t)T * slices;
  const int n = __builtin_amdgcn_readfirstlane(*num_recv);
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // unit gw < half: receive row r, slice gw - r * slices; else token gw - half
  auto move = [&](int64_t gw, int64_t r) {
    if (gw < half) {
      const int64_t c = (gw - r * slices) * kWave + lane;
      if (r >= n) return;
      const int64_t t = __builtin_amdgcn_readfirstlane(meta[r * (K + 2)]);
      if (t < 0 || t >= T || c >= row_chunks) return;
      const u32x4 v = __builtin_nontemporal_load(y + r * row_chunks + c);
      put_row_chunk<WIDE, FP32>(v, bias, t, row_chunks, c, out, stream_out);
    } else {
      const int64_t t = gw - half;
      bool any = false;
      for (int k = lane; k < K; k += kWave) any |= dst_slot[t * K + k] >= 0;
      if (ballot(any) != 0) return;  // received: written by its receive row
      for (int64_t c = lane; c < row_chunks; c += kWave)
        put_row_chunk<WIDE, FP32>(zero, bias, t, row_chunks, c, out, stream_out);
    }
  };
  if constexpr (WIDE) {  // one unit per wave, all of them in this launch (half + T < 2^26)
    const uint32_t w = blockIdx.x * (uint32_t)wpb + wave_in_block;
    if (w >= (uint32_t)(half + T)) return;
    move(w, fast_div_apply(w, by_slices));
  } else {
    const int64_t stride = (int64_t)gridDim.x * wpb;
    for (int64_t gw = (int64_t)blockIdx.x * wpb + wave_in_block; gw < half + T; gw += stride)
      move(gw, gw / slices);
  }
}

// Output rows (bytes, at most T rows) above which uncapped launches store
// them non-temporally (store_out_row): half of the 256 MiB last-level cache.
constexpr int64_t kCachedRowsBytes = int64_t(128) << 20;

// Uncapped (WIDE): one launch with one wave per unit and 32-bit indices,
// which needs units <= kMaxLaunchUnits (4.7M tokens at 14 slices per row).
// Capped, or beyond that size: one launch of at most `cap` (or 2^22)
// workgroups whose waves loop, with non-temporal stores.
template <bool WIDE>
int dispatch_compact_launch(const CompactDispatchArgs &a, int64_t units, int cap,
                            int64_t row_chunks) {
  const WaveGrid g = WIDE ? wave_grid(units, 0, 1 << 24) : wave_grid(units, cap, 1 << 22);
  ep_dispatch_compact_rows<WIDE><<<g.blocks, g.threads, 0, a.stream>>>(
      (const u32x4 *)a.x, row_chunks, a.x_scales, a.scale_cols, a.topk_idx, a.topk_weights,
      a.dst_slot, a.meta, a.num_recv, a.T, a.K, (u32x4 *)a.recv_x, a.recv_scales,
      a.recv_topk_idx, a.recv_topk_weights,
      fast_div((uint32_t)((row_chunks + kWave - 1) / kWave)),
      (int64_t)a.T * row_chunks * 16 > kCachedRowsBytes);
  return launch_status();
}

template <bool WIDE, bool FP32>
int combine_compact_launch(const CompactCombineArgs &a, int64_t units, int cap,
                           int64_t row_chunks) {
  const WaveGrid g = WIDE ? wave_grid(units, 0, 1 << 24) : wave_grid(units, cap, 1 << 22);
  ep_combine_compact_rows<WIDE, FP32><<<g.blocks, g.threads, 0, a.stream>>>(
      (const u32x4 *)a.y, row_chunks, (const u32x4 *)a.bias, a.dst_slot, a.meta, a.num_recv,
      a.T, a.K, (u32x4 *)a.out, fast_div((uint32_t)((row_chunks + kWave - 1) / kWave)),
      (int64_t)a.T * row_chunks * 16 > kCachedRowsBytes);
  return launch_status();
}

}  // namespace

int launch_dispatch_compact(const CompactDispatchArgs &a) {
  if (a.T == 0) return 0;
  const int64_t row_chunks = a.row_bytes / 16;
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int cap = stream_workgroup_limit(a.stream);
  const int64_t units = (int64_t)a.T * slices;
  return cap > 0 || units > kMaxLaunchUnits
             ? dispatch_compact_launch<false>(a, units, cap, row_chunks)
             : dispatch_compact_launch<true>(a, units, 0, row_chunks);
}

int launch_combine_compact(const CompactCombineArgs &a) {
  if (a.T == 0) return 0;
  const int64_t row_chunks = a.row_bytes / 16;
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int cap = stream_workgroup_limit(a.stream);
  const int64_t units = (int64_t)a.T * (slices + 1);
  const bool wide = cap == 0 && units <= kMaxLaunchUnits;
  if (a.fp32)
    return wide ? combine_compact_launch<true, true>(a, units, 0, row_chunks)
                : combine_compact_launch<false, true>(a, units, cap, row_chunks);
  return wide ? combine_compact_launch<true, false>(a, units, 0, row_chunks)
              : combine_compact_launch<false, false>(a, units, cap, row_chunks);
}

}  // namespace ep
