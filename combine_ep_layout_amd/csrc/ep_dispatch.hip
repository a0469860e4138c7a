// Dispatch in the expand layout for gfx950: expand_x[dst_slot[t, k]] = x[t]
// for every unmasked (t, k), with the fp8 scale row and the router weight
// travelling alongside.
//
// Follows "MORI JIT v2", section 3.7 (dispatch only moves its payload, never
// does arithmetic on elements; fp8 / fp4 arrive quantised and travel as
// one-byte elements) and the DeepEP overall-architecture page, dispatch
// data-flow figure (copy epilogue writing token data plus scale factors).
//
// Design (MI355X): the pass is HBM-bound on its writes (read T rows, write
// T*K rows). One wave64 moves one 1 KiB slice of one (token, k) row: a
// 16-byte load per lane from x and one 16-byte store per lane into the
// expand row, whose address is wave-uniform (the slot is loaded once and made
// scalar with readfirstlane). The store is non-temporal at device scope
// (RowStore::kNtDevice): expand rows are not read again by this pass. Waves are
// ordered token-major, then k, then slice, or, given the layout's dispatch
// plan, by ascending slot within each tile of tokens, then slice; either way
// each destination row is written front to back by consecutive waves, and
// the K waves that need the same source slice run on the same XCD, so x is
// read from HBM about once. Row bytes and K are template constants.
//
// When x is too large to stay in the last-level cache, the K waves that need
// one source slice all wait on the same HBM read, and few distinct bytes of x
// are in flight: the per-(token, k) wave order drops to about 3.3 TB/s. A
// second kernel then has one wave load the slice once and store it to a
// group of F of the token's entries (F = 4 for K = 8), so each wave in flight
// carries F times the writes per read (about 5.2 TB/s at 24576 tokens, and
// no loss on a cold x at 4096 tokens: 109 against 143 us).
//
// Under a workgroup cap (CU-limited mode) a compute unit's own memory path,
// not HBM, is the limit, so the same copy runs with F = K: one wave per
// (token, slice) loads the slice once and stores it to all K destinations,
// (K + 1) KiB per K KiB written instead of 2K KiB.
#include <algorithm>

#include "ep_device.hpp"
#include "ep_launch.hpp"

namespace ep {
namespace {


// Blocks run on the 8 XCDs round-robin (block b on XCD b % 8). Renumbering
// them so that each XCD gets one contiguous eighth of the work keeps the K
// waves that copy the same source slice on one XCD, where all but the first
// read it from that XCD's L2. The renumbering is a permutation only when the
// grid is a multiple of 8: the launcher pads the grid to one. xcd_wave gives
// the calling wave's index in a launch of kDefaultThreads-thread workgroups
// under that renumbering, in 32 bits (grids of at most 2^24 workgroups).
constexpr int kXcds = 8;
__device__ __forceinline__ uint32_t xcd_wave() {
  const uint32_t nb = gridDim.x, b = blockIdx.x;
  return ((b % kXcds) * (nb / kXcds) + b / kXcds) * (kDefaultThreads / kWave) +
         __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

// Moves slice `slice` of x[t] (entry tk) to expand row d; slice 0 also
// carries the scale row and the router weight.
template <int ROWB, int SCB>
__device__ __forceinline__ void copy_slice(const u32x4 *__restrict__ x,
                                           const u32x4 *__restrict__ x_scales,
                                           const float *__restrict__ topk_weights, int t,
                                           int tk, int slice, int d, int lane,
                                           u32x4 *__restrict__ expand_x,
                                           u32x4 *__restrict__ expand_scales,
                                           float *__restrict__ expand_weights) {
  constexpr int CH = ROWB / 16;
  constexpr int SCH = SCB / 16;
  const int i = slice * kWave + lane;
  if (CH % kWave == 0 || i < CH)
    store_row<RowStore::kNtDevice>(x[(int64_t)t * CH + i], expand_x + (int64_t)d * CH, ROWB,
                                   i * 16);
  if (slice == 0) {
    if (SCH > 0 && lane < SCH)
      __builtin_nontemporal_store(x_scales[(int64_t)t * SCH + lane],
                                  expand_scales + (int64_t)d * SCH + lane);
    if (expand_weights != nullptr && lane == 0) expand_weights[d] = topk_weights[tk];
  }
}

// One wave per (token, k, 1 KiB slice of the row): it reads 16 bytes per lane
// of x[t] and writes them to expand_x[dst_slot[t, k]] with one non-temporal
// store. Consecutive waves write consecutive KiB of one destination row, the
// order in which HBM absorbs writes fastest (a wave that scatters to K rows
// in turn is slower). The fp8 scale row and the router weight travel with
// slice 0. Entries are taken token-major, or with PLANNED in the order of the
// layout's dispatch plan. Inside each tile of tokens the plan lists entries by
// ascending slot, so consecutive entries are consecutive rows of one expert's
// segment. Runs of about 4 rows at 128 tokens per tile make HBM absorb the
// writes faster (prefill copy 79 against 85 us), and a tile's x rows (1.8 MB)
// stay in the XCD's L2 for its K re-reads.
// PLANNED: each wave moves exactly one unit, slice (w mod SLICES) of plan
// entry entry0 + w / SLICES, w its wave index in the launch (w < units); the
// host issues further launches past the grid limit. That walk's cost is its
// per-wave scalar work: one scalar unit serves a compute unit's four SIMDs,
// and at prefill each compute unit runs about 1800 of these waves. So its
// index arithmetic is 32-bit (entries, slots and a launch's units all fit),
// and without a loop the compiler loads each kernel argument where it is
// first used instead of all of them up front (prefill copy 75.1 against 80.5
// us with a grid-stride loop and 64-bit indices; MI355X, events). The
// token-major walk measured the other way (prefill 86.6 against 83.5 us,
// mori_default 22.9 against 21.7 in that form), so it keeps one launch
// whose waves loop over all units (entry0 = 0).
// DT (the EP_* dtype) only names the kernel: every dtype moves bytes, so
// instances with equal ROWB and SCB have the same body.
template <int DT, int ROWB, int SCB, int K, bool PLANNED>
__global__ __launch_bounds__(kDefaultThreads) void ep_dispatch_expand(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ x_scales,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ dst_slot,
    const int2 *__restrict__ plan, int entries, int capacity, u32x4 *__restrict__ expand_x,
    u32x4 *__restrict__ expand_scales, float *__restrict__ expand_weights, int entry0,
    int units) {
  constexpr int CH = ROWB / 16;                    // 16-byte chunks per row
  constexpr int SLICES = (CH + kWave - 1) / kWave;  // 1 KiB slices per row
  constexpr int SCH = SCB / 16;                    // 16-byte chunks per scale row
  static_assert(ROWB % 16 == 0 && SCB % 16 == 0 && SCH <= kWave, "row geometry");
  static_assert(K >= 1 && K <= kWave, "topk must fit one wavefront");
  if constexpr (PLANNED) {
    const uint32_t w = xcd_wave();
    if (w >= (uint32_t)units) return;
    const uint32_t jl = w / SLICES;
    const int slice = (int)(w - jl * SLICES);
    const int2 pe = plan[entry0 + (int)jl];
    const int tk = __builtin_amdgcn_readfirstlane(pe.x);  // flat (token, k)
    const int d = __builtin_amdgcn_readfirstlane(pe.y);
    if ((uint32_t)tk >= (uint32_t)entries || (uint32_t)d >= (uint32_t)capacity) return;
    copy_slice<ROWB, SCB>(x, x_scales, topk_weights, (int)((uint32_t)tk / K), tk, slice, d,
                          lane_id(), expand_x, expand_scales, expand_weights);
  } else {
    const int lane = lane_id();
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    constexpr int wpb = kDefaultThreads / kWave;
    const int64_t nb = gridDim.x, b = blockIdx.x;
    const int64_t total = (int64_t)entries * SLICES;
    const int64_t stride = nb * wpb;
    for (int64_t gw = ((b % kXcds) * (nb / kXcds) + b / kXcds) * wpb + wave_in_block; gw < total;
         gw += stride) {
      const int64_t tk = gw / SLICES;  // flat (token, k)
      const int slice = (int)(gw - tk * SLICES);
      const int d = __builtin_amdgcn_readfirstlane(dst_slot[tk]);
      if (d < 0 || d >= capacity) continue;
      copy_slice<ROWB, SCB>(x, x_scales, topk_weights, (int)(tk / K), (int)tk, slice, d, lane,
                            expand_x, expand_scales, expand_weights);
    }
  }
}

// Copies slice `slice` of token t's row to the destination rows of the F
// entries k0 .. k0 + F - 1 (masked entries skipped); slice 0 also carries
// the scale row and each entry's router weight. Slots, slice and scale row
// are loaded first and waited for once, so the F stores leave back to back.
template <int ROWB, int SCB, int K, int F, RowStore P>
__device__ __forceinline__ void copy_slice_to_group(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ x_scales,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ dst_slot, int t,
    int k0, int slice, int capacity, u32x4 *__restrict__ expand_x,
    u32x4 *__restrict__ expand_scales, float *__restrict__ expand_weights) {
  constexpr int CH = ROWB / 16;
  constexpr int SCH = SCB / 16;
  static_assert(ROWB % 16 == 0 && SCB % 16 == 0 && SCH <= kWave, "row geometry");
  static_assert(F >= 1 && F <= K && K % F == 0 && K <= kWave, "entry group");
  const int lane = lane_id();
  const int tk0 = t * K + k0;  // below num_tokens * topk, an int32
  const int i = slice * kWave + lane;
  const bool in_row = CH % kWave == 0 || i < CH;
  u32x4 v = {0u, 0u, 0u, 0u}, sc = {0u, 0u, 0u, 0u};
  if (in_row) v = x[(int64_t)t * CH + i];
  if (SCH > 0 && slice == 0 && lane < SCH) sc = x_scales[(int64_t)t * SCH + lane];
  // every lane reads a slot (lanes past F repeat entry k0) so that no branch
  // separates this load from the ones above and all are in flight together
  int my_d = dst_slot[tk0 + (lane < F ? lane : 0)];
  wait_vector_memory();
  if (lane >= F || (uint32_t)my_d >= (uint32_t)capacity) my_d = -1;
#pragma unroll
  for (int j = 0; j < F; ++j) {
    const int d = read_lane(my_d, j);
    if (d < 0) continue;
    if (in_row) store_row<P>(v, expand_x + (int64_t)d * CH, ROWB, i * 16);
    if (slice == 0) {
      if (SCH > 0 && lane < SCH)
        __builtin_nontemporal_store(sc, expand_scales + (int64_t)d * SCH + lane);
      if (expand_weights != nullptr && lane == 0) expand_weights[d] = topk_weights[tk0 + j];
    }
  }
}

// Uncapped, x larger than the cache can hold: one wave per (token, group of
// F entries, 1 KiB slice), ordered token-major, then group, then slice, with
// the blocks of one XCD contiguous as in ep_dispatch_expand. Each wave moves
// one unit: slice (w mod SLICES) of group group0 + w / SLICES, w its wave
// index in the launch (w < units), with 32-bit index arithmetic as in
// ep_dispatch_expand.
template <int DT, int ROWB, int SCB, int K, int F>
__global__ __launch_bounds__(kDefaultThreads) void ep_dispatch_grouped(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ x_scales,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ dst_slot, int capacity,
    u32x4 *__restrict__ expand_x, u32x4 *__restrict__ expand_scales,
    float *__restrict__ expand_weights, int group0, int units) {
  constexpr int SLICES = (ROWB / 16 + kWave - 1) / kWave;
  constexpr uint32_t KG = K / F;  // entry groups per token
  const uint32_t w = xcd_wave();
  if (w >= (uint32_t)units) return;
  const uint32_t gl = w / SLICES;
  const int slice = (int)(w - gl * SLICES);
  const uint32_t tg = (uint32_t)group0 + gl;  // flat (token, group)
  const uint32_t t = tg / KG;
  const int g = (int)(tg - t * KG);
  copy_slice_to_group<ROWB, SCB, K, F, RowStore::kNtDevice>(x, x_scales, topk_weights, dst_slot,
                                                            (int)t, g * F, slice, capacity,
                                                            expand_x, expand_scales,
                                                            expand_weights);
}

// Under a workgroup cap: one wave per (token, 1 KiB slice), all K entries.
template <int DT, int ROWB, int SCB, int K>
__global__ __launch_bounds__(kCappedThreads) void ep_dispatch_fanout(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ x_scales,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ dst_slot, int T,
    int64_t capacity, u32x4 *__restrict__ expand_x, u32x4 *__restrict__ expand_scales,
    float *__restrict__ expand_weights) {
  constexpr int SLICES = (ROWB / 16 + kWave - 1) / kWave;
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  constexpr int wpb = kCappedThreads / kWave;  // launched under a cap only
  const int64_t total = (int64_t)T * SLICES;
  const int64_t stride = (int64_t)gridDim.x * wpb;
  const int cap32 = (int)(capacity < INT32_MAX ? capacity : INT32_MAX);
  for (int64_t gw = (int64_t)blockIdx.x * wpb + wave_in_block; gw < total; gw += stride) {
    const int t = (int)(gw / SLICES);
    const int slice = (int)(gw - (int64_t)t * SLICES);
    copy_slice_to_group<ROWB, SCB, K, K, RowStore::kNt>(x, x_scales, topk_weights, dst_slot, t, 0,
                                                        slice, cap32, expand_x, expand_scales,
                                                        expand_weights);
  }
}

// Bytes of x above which the uncapped launch uses ep_dispatch_grouped: half
// of MI355X's 256 MiB last-level cache. Below it x, written by the kernel
// before dispatch, is normally still cached and the per-(token, k) order is
// fastest (87 against 95 us at 4096 tokens); above it x rarely survives
// beside the other traffic, and past the full 256 MiB it never does.
constexpr int64_t kCachedXBytes = int64_t(128) << 20;

template <int DT, int ROWB, int SCB, int K>
int dispatch_impl(const DispatchArgs &a) {
  if (a.T == 0) return 0;
  constexpr int SLICES = (ROWB / 16 + kWave - 1) / kWave;
  constexpr int F = K % 4 == 0 ? 4 : K % 3 == 0 ? 3 : K % 2 == 0 ? 2 : 1;  // entries per wave
  const bool fwd_w = a.topk_weights != nullptr && a.expand_weights != nullptr;
  const u32x4 *x = (const u32x4 *)a.x, *xs = (const u32x4 *)a.x_scales;
  u32x4 *ex = (u32x4 *)a.expand_x, *es = (u32x4 *)a.expand_scales;
  float *ew = fwd_w ? a.expand_weights : nullptr;
  const int cap = stream_workgroup_limit(a.stream);
  if (cap > 0) {
    const WaveGrid g = wave_grid((int64_t)a.T * SLICES, cap, 1 << 24);
    ep_dispatch_fanout<DT, ROWB, SCB, K><<<g.blocks, kCappedThreads, 0, a.stream>>>(
        x, xs, a.topk_weights, a.dst_slot, a.T, a.capacity, ex, es, ew);
    return launch_status();
  }
  // Uncapped: one wave per unit, in launches of whole entries (or entry
  // groups) of at most kMaxLaunchUnits units. Slots are int32, so a capacity
  // beyond INT32_MAX admits them all.
  const int cap32 = (int)std::min<int64_t>(a.capacity, INT32_MAX);
  if constexpr (F > 1) {
    if ((int64_t)a.T * ROWB > kCachedXBytes) {
      const int groups = a.T * (K / F);
      constexpr int kLaunchGroups = (int)(kMaxLaunchUnits / SLICES);
      for (int g0 = 0; g0 < groups; g0 += std::min(kLaunchGroups, groups - g0)) {
        const int units = std::min(kLaunchGroups, groups - g0) * SLICES;
        const WaveGrid g = wave_grid(units, 0, 1 << 24, kXcds);
        ep_dispatch_grouped<DT, ROWB, SCB, K, F><<<g.blocks, kDefaultThreads, 0, a.stream>>>(
            x, xs, a.topk_weights, a.dst_slot, cap32, ex, es, ew, g0, units);
        if (int r = launch_status()) return r;  // before the next launch
      }
      return 0;
    }
  }
  const int entries = a.T * K;  // at most INT32_MAX (checked by the C ABI)
  if (a.plan == nullptr) {  // one launch; its waves loop past the grid limit
    const WaveGrid g = wave_grid((int64_t)entries * SLICES, 0, 1 << 24, kXcds);
    ep_dispatch_expand<DT, ROWB, SCB, K, false><<<g.blocks, kDefaultThreads, 0, a.stream>>>(
        x, xs, a.topk_weights, a.dst_slot, nullptr, entries, cap32, ex, es, ew, 0, 0);
    return launch_status();
  }
  constexpr int kLaunchEntries = (int)(kMaxLaunchUnits / SLICES);
  for (int e0 = 0; e0 < entries; e0 += std::min(kLaunchEntries, entries - e0)) {
    const int units = std::min(kLaunchEntries, entries - e0) * SLICES;
    const WaveGrid g = wave_grid(units, 0, 1 << 24, kXcds);
    ep_dispatch_expand<DT, ROWB, SCB, K, true><<<g.blocks, kDefaultThreads, 0, a.stream>>>(
        x, xs, a.topk_weights, a.dst_slot, (const int2 *)a.plan, entries, cap32, ex, es, ew, e0,
        units);
    if (int r = launch_status()) return r;  // before the next launch
  }
  return 0;
}

// Row and scale-row bytes per dtype. hidden counts elements for bf16, fp32
// and fp8, bytes for fp4x2; a scale row holds one fp32 per 128 elements.
template <int DT, int H, bool SCALES, int K>
int dispatch_dt(const DispatchArgs &a) {
  constexpr int ELT_BYTES_X2 = DT == 0 ? 4 : DT == 1 ? 8 : 2;  // twice the bytes per hidden unit
  constexpr int ROWB = H * ELT_BYTES_X2 / 2;
  constexpr int ELEMS = DT == 3 ? 2 * H : H;
  constexpr int SCB = SCALES ? (ELEMS / 128) * 4 : 0;
  return dispatch_impl<DT, ROWB, SCB, K>(a);
}

}  // namespace

#define EP_DISPATCH_K(K) \
  case K:                \
    return dispatch_dt<DT, H, SCALES, K>(a);

template <int DT, int H, bool SCALES>
static int dispatch_k(const DispatchArgs &a) {
  switch (a.K) { EP_FOR_EACH_TOPK(EP_DISPATCH_K) default: return -2; }
}

#define EP_DISPATCH_H_PLAIN(H) \
  case H:                      \
    return dispatch_k<DT, H, false>(a);
#define EP_DISPATCH_H_BYTES(H)                                                         \
  case H:                                                                              \
    return a.x_scales ? dispatch_k<DT, H, true>(a) : dispatch_k<DT, H, false>(a);

template <int DT>
static int dispatch_plain(const DispatchArgs &a);
template <>
int dispatch_plain<0>(const DispatchArgs &a) {
  constexpr int DT = 0;
  switch (a.H) { EP_FOR_EACH_HIDDEN_BF16(EP_DISPATCH_H_PLAIN) default: return -2; }
}
template <>
int dispatch_plain<1>(const DispatchArgs &a) {
  constexpr int DT = 1;
  switch (a.H) { EP_FOR_EACH_HIDDEN_FP32(EP_DISPATCH_H_PLAIN) default: return -2; }
}
static int dispatch_fp8(const DispatchArgs &a) {
  constexpr int DT = 2;
  switch (a.H) { EP_FOR_EACH_HIDDEN_FP8(EP_DISPATCH_H_BYTES) default: return -2; }
}
static int dispatch_fp4x2(const DispatchArgs &a) {
  constexpr int DT = 3;
  switch (a.H) { EP_FOR_EACH_HIDDEN_FP4X2(EP_DISPATCH_H_BYTES) default: return -2; }
}

int launch_dispatch(const DispatchArgs &a) {
  switch (a.dtype) {
    case 0: return dispatch_plain<0>(a);
    case 1: return dispatch_plain<1>(a);
    case 2: return dispatch_fp8(a);
    case 3: return dispatch_fp4x2(a);
    default: return -2;
  }
}

#define EP_IS(V) \
  case V:        \
    return true;

static bool has_topk(int K) {
  switch (K) { EP_FOR_EACH_TOPK(EP_IS) default: return false; }
}

bool has_layout(int K) { return has_topk(K); }

bool has_dispatch(int H, int K, int dtype) {
  if (!has_topk(K)) return false;
  switch (dtype) {
    case 0: switch (H) { EP_FOR_EACH_HIDDEN_BF16(EP_IS) default: return false; }
    case 1: switch (H) { EP_FOR_EACH_HIDDEN_FP32(EP_IS) default: return false; }
    case 2: switch (H) { EP_FOR_EACH_HIDDEN_FP8(EP_IS) default: return false; }
    case 3: switch (H) { EP_FOR_EACH_HIDDEN_FP4X2(EP_IS) default: return false; }
    default: return false;
  }
}

bool has_combine(int H, int K, int dtype) {
  if (!has_topk(K)) return false;
  switch (dtype) {
    case 0: switch (H) { EP_FOR_EACH_HIDDEN_BF16(EP_IS) default: return false; }
    case 1: switch (H) { EP_FOR_EACH_HIDDEN_FP32(EP_IS) default: return false; }
    default: return false;
  }
}

}  // namespace ep
