// Gather combine for gfx950: out[t] = sum_k w[t,k] * y[dst_slot[t,k]] (+ bias[t])
// with binary32 accumulation in k order, the bias added last, and a store in
// the rows' type (bf16: round to nearest even).
//
// Follows the DeepEP overall-architecture page, combine data-flow figure
// (the reduce epilogue weights each expert output by topk_weights, adds a
// bias and writes back in token order) and "MORI JIT v2", section 3.7
// (combine reduces bf16 or fp32 rows; byte dtypes are rejected upstream).
//
// Design (MI355X): HBM-bound (read T*K rows, write T rows, about 1 flop per
// byte). A wave loads its token's K slots and weights with K lanes and
// broadcasts them with readlane, so row addresses are wave-uniform. Two
// kernels cut the work differently:
//   - ep_combine_stream (uncapped, at least 1024 tokens, rows of 4 to 14
//     16-byte chunks per lane): one wave per token keeps the whole output row
//     in binary32 and walks the K rows in k order with the next row's loads
//     in flight. Reading each row whole is the gather order HBM serves best
//     (measured on MI355X, pure gathers of 8 rows of 14 KiB: 85 us per 4096
//     tokens whole-row, 89 us in 2 KiB pieces); prefill combine 92 against
//     96 us.
//   - ep_combine_gather (otherwise): a row is cut into slices of two 16-byte
//     chunks per lane (2 KiB); one wave owns one (token, slice), so a
//     14,336-byte row is served by 7 waves, and issues all K*2 loads (16 KiB)
//     before folding. Small batches need these many short waves to fill the
//     chip (128 tokens: 8 against 12 us for one wave per token).
// Loads are non-temporal: expert outputs are read once. Output rows are
// stored at device scope and kept (RowStore::kDevice; under a workgroup cap,
// non-temporally): at 59 MB they fit the last-level cache, which absorbs
// them faster than writes streamed to HBM between the loads (prefill 86.9
// against 91.6 us), and the next layer reads them from there. Both kernels
// fold the same way: products and sums
// are rounded separately (contraction off), in k order, so the result is a
// pure function of the inputs; the final pack uses the hardware binary32 ->
// bf16 convert, which rounds to nearest even.
#include <algorithm>

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

// Waves per token and 16-byte chunks per lane per pass for a row of CH chunks:
// each wave takes two chunks per lane (2 KiB of each of the K rows) when the
// row divides evenly, else one; small rows keep one wave per token.
template <int CH>
struct CombineGeometry {
  static constexpr int CPL = (CH + kWave - 1) / kWave;  // chunks per lane for a whole row
  static constexpr int G = CPL % 2 == 0 ? 2 : 1;         // chunks per lane per wave
  static constexpr int SPLIT = CPL / G;                  // waves per token
};

// Element type of the rows: EP_BF16 (0) packs 8 values per 16-byte chunk,
// EP_FP32 (1) packs 4.
template <int DT>
struct Elem {
  static constexpr int BYTES = DT == 0 ? 2 : 4;
  static constexpr int PER_CHUNK = 16 / BYTES;
  // Value j of a chunk, widened to binary32 (exact).
  static __device__ __forceinline__ float get(const u32x4 &c, int j) {
    if constexpr (DT == 0) {
      const uint32_t word = c[j >> 1];
      return __uint_as_float((j & 1) ? (word & 0xffff0000u) : (word << 16));
    } else {
      return __uint_as_float(c[j]);
    }
  }
  // A chunk of sums stored in the row's type (bf16: round to nearest even).
  static __device__ __forceinline__ u32x4 put(const float (&acc)[PER_CHUNK]) {
    u32x4 r;
    if constexpr (DT == 0) {
      r[0] = pack_bf16x2(acc[0], acc[1]);
      r[1] = pack_bf16x2(acc[2], acc[3]);
      r[2] = pack_bf16x2(acc[4], acc[5]);
      r[3] = pack_bf16x2(acc[6], acc[7]);
    } else {
      r[0] = __float_as_uint(acc[0]);
      r[1] = __float_as_uint(acc[1]);
      r[2] = __float_as_uint(acc[2]);
      r[3] = __float_as_uint(acc[3]);
    }
    return r;
  }
};

// Loads the wave's slice (G chunks per lane) of each of the K rows and folds
// them in k order into acc. ALL_VALID: every slot is a real row, so the
// loads are straight-line code and each row is consumed as soon as its loads
// land; otherwise rows with a negative slot d[k] are skipped by the fold,
// and their loads read src[k], another row of the same token, so that the
// loads stay straight-line code (no partly loaded register array).
template <int DT, int CH, int K, int G, bool ALL_VALID>
__device__ __forceinline__ void gather_fold(const u32x4 *__restrict__ y, const int (&src)[K],
                                            const int (&d)[K], const float (&wk)[K], int c0,
                                            int lane, float (&acc)[G][Elem<DT>::PER_CHUNK]) {
#pragma clang fp contract(off)
  constexpr int PC = Elem<DT>::PER_CHUNK;
  u32x4 v[K][G];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const u32x4 *row = y + (int64_t)src[k] * CH;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = (c0 + g) * kWave + lane;
      if (CH % kWave == 0 || i < CH) v[k][g] = __builtin_nontemporal_load(row + i);
    }
  }
  // Keep every load above the arithmetic: the scheduler would otherwise sink
  // some of them below it to save registers, halving the bytes in flight.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < PC; ++j) acc[g][j] = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {  // fixed k order
    if (!ALL_VALID && d[k] < 0) continue;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int j = 0; j < PC; ++j) {
        const float p = wk[k] * Elem<DT>::get(v[k][g], j);
        acc[g][j] = acc[g][j] + p;
      }
    }
  }
}

// NT threads per workgroup: 256 normally; 1024 under a workgroup cap (16
// waves, 16 KiB of loads in flight each, on the one compute unit the
// workgroup occupies; at most 128 registers per lane).
constexpr int kCombineCappedThreads = kCappedThreads;

template <int DT, int H, int K, bool BIAS, int NT>
__global__ __launch_bounds__(NT) void ep_combine_gather(
    const u32x4 *__restrict__ y, const float *__restrict__ topk_weights,
    const u32x4 *__restrict__ bias, const int32_t *__restrict__ dst_slot, int T,
    int64_t capacity, u32x4 *__restrict__ out, int t0, int units) {
  constexpr int CH = H * Elem<DT>::BYTES / 16;  // 16-byte chunks per row
  constexpr int PC = Elem<DT>::PER_CHUNK;
  using Geo = CombineGeometry<CH>;
  constexpr int G = Geo::G, SPLIT = Geo::SPLIT;
  static_assert((H * Elem<DT>::BYTES) % 16 == 0, "row geometry");
  static_assert(K >= 1 && K <= kWave, "topk must fit one wavefront");

  const int lane = lane_id();
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  constexpr int wpb = NT / kWave;
  // Token t, slices from chunk c0 (per lane) on.
  auto unit = [&](const int t, const int c0) {
    int my_dst = -1;
    float my_w = 0.f;
    if (lane < K) {
      my_dst = dst_slot[(int64_t)t * K + lane];
      if (my_dst >= capacity) my_dst = -1;
      my_w = topk_weights ? topk_weights[(int64_t)t * K + lane] : 1.0f;
    }
    const uint64_t valid = ballot(lane < K && my_dst >= 0);
    int d[K];
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      d[k] = read_lane(my_dst, k);
      wk[k] = read_lane(my_w, k);
    }
    // Expert outputs are read exactly once: non-temporal loads keep them
    // from displacing useful lines in the caches.
    float acc[G][PC];
    if (valid == (K == 64 ? ~0ull : (1ull << K) - 1)) {
      gather_fold<DT, CH, K, G, true>(y, d, d, wk, c0, lane, acc);
    } else if (valid != 0) {  // masked slots load a valid row of the token, unused
      const int any = read_lane(my_dst, __builtin_ctzll(valid));
      int src[K];
#pragma unroll
      for (int k = 0; k < K; ++k) src[k] = d[k] >= 0 ? d[k] : any;
      gather_fold<DT, CH, K, G, false>(y, src, d, wk, c0, lane, acc);
    } else {  // no expert output for this token: the sum of no terms
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < PC; ++j) acc[g][j] = 0.0f;
    }

    u32x4 *o = out + (int64_t)t * CH;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = (c0 + g) * kWave + lane;
      if (CH % kWave == 0 || i < CH) {
        if constexpr (BIAS) {  // added once, after the k-order sum
#pragma clang fp contract(off)
          const u32x4 b = bias[(int64_t)t * CH + i];
#pragma unroll
          for (int j = 0; j < PC; ++j) acc[g][j] = acc[g][j] + Elem<DT>::get(b, j);
        }
        store_row<NT == kDefaultThreads ? RowStore::kDevice : RowStore::kNt>(
            Elem<DT>::put(acc[g]), o, CH * 16, i * 16);
      }
    }
  };
  if constexpr (NT == kDefaultThreads) {
    // Uncapped: wave w moves unit w of tokens [t0, t0 + units / SPLIT), with
    // 32-bit indices (the index arithmetic sits on the wave's path to its
    // first loads).
    const uint32_t w = blockIdx.x * (uint32_t)wpb + wave_in_block;
    if (w >= (uint32_t)units) return;
    const uint32_t tl = w / SPLIT;
    unit(t0 + (int)tl, (int)(w - tl * SPLIT) * G);
  } else {  // under a cap the waves loop over every token
    const int64_t stride = (int64_t)gridDim.x * wpb;
    for (int64_t gw = (int64_t)blockIdx.x * wpb + wave_in_block; gw < (int64_t)T * SPLIT;
         gw += stride) {
      const int t = (int)(gw / SPLIT);
      unit(t, (int)(gw - (int64_t)t * SPLIT) * G);
    }
  }
}

// Pieces of a row for ep_combine_stream: rows of whole chunks per lane, cut
// into the fewest equal pieces of at most 14 chunks per lane (the registers
// of one binary32 piece plus two rows in flight, 254 of them at 14).
template <int CH>
struct StreamGeometry {
  static constexpr int ROW_CPL = CH / kWave;
  static constexpr int PIECES = ROW_CPL > 14 ? (ROW_CPL + 13) / 14 : 1;
  static constexpr int CPL = ROW_CPL / PIECES;  // chunks per lane per piece
  static constexpr bool OK = CH % kWave == 0 && ROW_CPL % PIECES == 0 && CPL >= 4;
};

// Row-streaming combine for rows of whole chunks per lane: one wave per token
// (per piece of at most 14 chunks per lane, for the widest fp32 rows) holds
// its part of the output row in binary32 (CPL chunks per lane) and walks the
// K expert rows in k order, with the next D - 1 rows' loads in flight while
// a row is folded. The fold is the same sequence of binary32 operations as
// ep_combine_gather's. Rows with a negative slot are skipped; their loads
// read another row of the token (src) so the loads stay straight-line code.
template <int DT, int CH, int CPL, int K, int D, bool ALL_VALID>
__device__ __forceinline__ void stream_fold(const u32x4 *__restrict__ y, const int (&src)[K],
                                            const int (&d)[K], const float (&wk)[K], int i0,
                                            float (&acc)[CPL][Elem<DT>::PER_CHUNK]) {
#pragma clang fp contract(off)
  constexpr int PC = Elem<DT>::PER_CHUNK;
  u32x4 buf[D][CPL];
#pragma unroll
  for (int r = 0; r < D; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      buf[r][c] = __builtin_nontemporal_load(y + (int64_t)src[r] * CH + i0 + c * kWave);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int j = 0; j < PC; ++j) acc[c][j] = 0.0f;
#pragma unroll
  for (int k = 0; k < K; ++k) {  // fixed k order
    if (ALL_VALID || d[k] >= 0) {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int j = 0; j < PC; ++j) {
          const float p = wk[k] * Elem<DT>::get(buf[k % D][c], j);
          acc[c][j] = acc[c][j] + p;
        }
    }
    if (k + D < K) {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        buf[k % D][c] = __builtin_nontemporal_load(y + (int64_t)src[k + D] * CH + i0 + c * kWave);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Fewest tokens for ep_combine_stream: one wave per token must fill the
// chip's 2048 wave slots at its two waves per SIMD.
constexpr int kStreamMinTokens = 1024;

// Output bytes above which ep_combine_stream stores its rows non-temporally:
// half of MI355X's 256 MiB last-level cache. Below it the kept rows are
// absorbed by that cache (prefill, 59 MB: 86.9 against 91.6 us; fp8_hot8 and
// binary32 rows, 117 MB: 167.4 against 177.2 us and 170.8 against 179.4);
// above it they only evict other lines (32K tokens, 470 MB: 731 against
// 753 us with them kept).
constexpr int64_t kCachedOutBytes = int64_t(128) << 20;

// stream_out: the output rows are larger than the last-level cache can keep
// beside the other traffic, so they are stored non-temporally at device scope
// (RowStore::kNtDevice) instead of kept (RowStore::kDevice); a wave-uniform
// branch around the stores.
template <int DT, int H, int K, bool BIAS>
__global__ __launch_bounds__(kDefaultThreads) void ep_combine_stream(
    const u32x4 *__restrict__ y, const float *__restrict__ topk_weights,
    const u32x4 *__restrict__ bias, const int32_t *__restrict__ dst_slot, int T,
    int64_t capacity, u32x4 *__restrict__ out, int stream_out) {
  constexpr int CH = H * Elem<DT>::BYTES / 16;
  constexpr int PC = Elem<DT>::PER_CHUNK;
  using Geo = StreamGeometry<CH>;
  constexpr int CPL = Geo::CPL, PIECES = Geo::PIECES;
  constexpr int D = K < 2 ? K : 2;  // rows in flight
  const int lane = lane_id();
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  constexpr int wpb = kDefaultThreads / kWave;
  const int64_t stride = (int64_t)gridDim.x * wpb;
  for (int64_t gw = (int64_t)blockIdx.x * wpb + wave_in_block; gw < (int64_t)T * PIECES;
       gw += stride) {
    const int64_t t = gw / PIECES;
    const int i0 = (int)(gw - t * PIECES) * CPL * kWave + lane;  // this lane's first chunk
    int my_dst = -1;
    float my_w = 0.f;
    if (lane < K) {
      my_dst = dst_slot[t * K + lane];
      if (my_dst >= capacity) my_dst = -1;
      my_w = topk_weights ? topk_weights[t * K + lane] : 1.0f;
    }
    const uint64_t valid = ballot(lane < K && my_dst >= 0);
    int d[K];
    float wk[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      d[k] = read_lane(my_dst, k);
      wk[k] = read_lane(my_w, k);
    }
    float acc[CPL][PC];
    if (valid == (K == 64 ? ~0ull : (1ull << K) - 1)) {
      stream_fold<DT, CH, CPL, K, D, true>(y, d, d, wk, i0, acc);
    } else if (valid != 0) {
      const int any = read_lane(my_dst, __builtin_ctzll(valid));
      int src[K];
#pragma unroll
      for (int k = 0; k < K; ++k) src[k] = d[k] >= 0 ? d[k] : any;
      stream_fold<DT, CH, CPL, K, D, false>(y, src, d, wk, i0, acc);
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
#pragma unroll
        for (int j = 0; j < PC; ++j) acc[c][j] = 0.0f;
    }
    u32x4 *o = out + t * CH;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int i = i0 + c * kWave;
      if constexpr (BIAS) {
#pragma clang fp contract(off)
        const u32x4 b = bias[t * CH + i];
#pragma unroll
        for (int j = 0; j < PC; ++j) acc[c][j] = acc[c][j] + Elem<DT>::get(b, j);
      }
      if (stream_out)
        store_row<RowStore::kNtDevice>(Elem<DT>::put(acc[c]), o, CH * 16, i * 16);
      else
        store_row<RowStore::kDevice>(Elem<DT>::put(acc[c]), o, CH * 16, i * 16);
    }
  }
}

template <int DT, int H, int K, int NT>
void combine_launch(const CombineArgs &a, const WaveGrid &g, int t0, int units) {
  if (a.bias)
    ep_combine_gather<DT, H, K, true, NT><<<g.blocks, NT, 0, a.stream>>>(
        (const u32x4 *)a.y, a.topk_weights, (const u32x4 *)a.bias, a.dst_slot, a.T, a.capacity,
        (u32x4 *)a.out, t0, units);
  else
    ep_combine_gather<DT, H, K, false, NT><<<g.blocks, NT, 0, a.stream>>>(
        (const u32x4 *)a.y, a.topk_weights, nullptr, a.dst_slot, a.T, a.capacity,
        (u32x4 *)a.out, t0, units);
}

template <int DT, int H, int K>
int combine_impl(const CombineArgs &a) {
  if (a.T == 0) return 0;
  constexpr int CH = H * Elem<DT>::BYTES / 16;
  const int cap = stream_workgroup_limit(a.stream);  // read once per launch
  if constexpr (StreamGeometry<CH>::OK) {
    if (a.T >= kStreamMinTokens && cap == 0) {
      // At most 2^24 workgroups (the grid limit of 2^32 threads); waves loop past it.
      const WaveGrid g = wave_grid((int64_t)a.T * StreamGeometry<CH>::PIECES, 0, 1 << 24);
      const int stream_out = (int64_t)a.T * CH * 16 > kCachedOutBytes;
      if (a.bias)
        ep_combine_stream<DT, H, K, true><<<g.blocks, kDefaultThreads, 0, a.stream>>>(
            (const u32x4 *)a.y, a.topk_weights, (const u32x4 *)a.bias, a.dst_slot, a.T,
            a.capacity, (u32x4 *)a.out, stream_out);
      else
        ep_combine_stream<DT, H, K, false><<<g.blocks, kDefaultThreads, 0, a.stream>>>(
            (const u32x4 *)a.y, a.topk_weights, nullptr, a.dst_slot, a.T, a.capacity,
            (u32x4 *)a.out, stream_out);
      return launch_status();
    }
  }
  constexpr int SPLIT = CombineGeometry<H * Elem<DT>::BYTES / 16>::SPLIT;
  if (cap > 0) {
    combine_launch<DT, H, K, kCombineCappedThreads>(
        a, wave_grid((int64_t)a.T * SPLIT, cap, 1 << 24, 1, kCombineCappedThreads), 0, 0);
    return launch_status();
  }
  // Uncapped: launches of whole tokens, at most kMaxLaunchUnits units each.
  constexpr int kLaunchTokens = (int)(kMaxLaunchUnits / SPLIT);
  for (int t0 = 0; t0 < a.T; t0 += std::min(kLaunchTokens, a.T - t0)) {
    const int units = std::min(kLaunchTokens, a.T - t0) * SPLIT;
    combine_launch<DT, H, K, kDefaultThreads>(a, wave_grid(units, 0, 1 << 24), t0, units);
    if (int r = launch_status()) return r;  // before the next launch
  }
  return 0;
}

}  // namespace

#define EP_COMBINE_K(K) \
  case K:               \
    return combine_impl<DT, H_, K>(a);

template <int DT, int H_>
static int combine_k(const CombineArgs &a) {
  switch (a.K) { EP_FOR_EACH_TOPK(EP_COMBINE_K) default: return -2; }
}

#define EP_COMBINE_H(H) \
  case H:               \
    return combine_k<DT, H>(a);

template <int DT>
static int combine_dt(const CombineArgs &a);
template <>
int combine_dt<0>(const CombineArgs &a) {
  constexpr int DT = 0;
  switch (a.H) { EP_FOR_EACH_HIDDEN_BF16(EP_COMBINE_H) default: return -2; }
}
template <>
int combine_dt<1>(const CombineArgs &a) {
  constexpr int DT = 1;
  switch (a.H) { EP_FOR_EACH_HIDDEN_FP32(EP_COMBINE_H) default: return -2; }
}

int launch_combine(const CombineArgs &a) {
  switch (a.dtype) {
    case 0: return combine_dt<0>(a);
    case 1: return combine_dt<1>(a);
    default: return -2;
  }
}

}  // namespace ep
