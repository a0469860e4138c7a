// Dispatch in the expand layout for gfx950: expand_x[dst_slot[t, k]] = x[t]
// for every unmasked (t, k), with the fp8 scale row and the router weight
// travelling alongside.
//
// Follows "MORI JIT v2", section 3.7 (dispatch only moves its payload, never
// does arithmetic on elements; fp8 / fp4 arrive quantised and travel as
// one-byte elements) and the DeepEP overall-architecture page, dispatch
// data-flow figure (copy epilogue writing token data plus scale factors).
//
// Design (MI355X): the pass is HBM-bound (read T rows, write T*K rows). A
// source row is cut into slices of two 16-byte chunks per lane (2 KiB); one
// wave64 owns one (token, slice): it loads its slice once into registers and
// writes it to each of the token's K destinations, so every x byte is read
// from HBM once and a 14,336-byte row is served by 7 waves. The K
// destination indices are loaded by K lanes and broadcast with readlane, so
// row addresses are wave-uniform (scalar base + lane offset) and every store
// instruction writes 1 KiB contiguous. Row bytes and K are template
// constants: the per-row loops unroll fully.
#include "ep_device.hpp"
#include "ep_launch.hpp"

namespace ep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // 4 waves, one token per wave at a time
constexpr int kWavesPerBlock = kThreads / kWave;

// Waves per token and 16-byte chunks per lane for a row of CH chunks: each
// wave moves two chunks per lane (2 KiB of the row) when the row divides
// evenly, else one; small rows keep one wave per token.
template <int CH>
struct DispatchGeometry {
  static constexpr int CPL = (CH + kWave - 1) / kWave;
  static constexpr int G = CPL % 2 == 0 ? 2 : 1;
  static constexpr int SPLIT = CPL / G;
};

template <int ROWB, int SCB, int K>
__global__ __launch_bounds__(kThreads) void ep_dispatch_expand(
    const u32x4 *__restrict__ x, const u32x4 *__restrict__ x_scales,
    const float *__restrict__ topk_weights, const int32_t *__restrict__ dst_slot, int T,
    int64_t capacity, u32x4 *__restrict__ expand_x, u32x4 *__restrict__ expand_scales,
    float *__restrict__ expand_weights) {
  constexpr int CH = ROWB / 16;  // 16-byte chunks per row
  using Geo = DispatchGeometry<CH>;
  constexpr int G = Geo::G, SPLIT = Geo::SPLIT;
  constexpr int SCH = SCB / 16;  // 16-byte chunks per scale row
  static_assert(ROWB % 16 == 0 && SCB % 16 == 0 && SCH <= kWave, "row geometry");
  static_assert(K >= 1 && K <= kWave, "topk must fit one wavefront");

  const int lane = lane_id();
  const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t first = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block;
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;

  for (int64_t gw = first; gw < (int64_t)T * SPLIT; gw += stride) {
    const int t = (int)(gw / SPLIT);
    const int part = (int)(gw - (int64_t)t * SPLIT);
    const int c0 = part * G;
    int my_dst = -1;
    if (lane < K) {
      my_dst = dst_slot[(int64_t)t * K + lane];
      if (my_dst >= capacity) my_dst = -1;
    }
    u32x4 v[G];
    const u32x4 *src = x + (int64_t)t * CH;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int i = (c0 + g) * kWave + lane;
      if (CH % kWave == 0 || i < CH) v[g] = src[i];
    }
    u32x4 s = {0u, 0u, 0u, 0u};
    const bool scale_lane = SCH > 0 && part == 0 && lane < SCH;
    if (scale_lane) s = x_scales[(int64_t)t * SCH + lane];
    // The expand buffer is written once and read by a later kernel:
    // non-temporal stores stream it to HBM without holding cache lines.
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int d = read_lane(my_dst, k);
      if (d < 0) continue;
      u32x4 *o = expand_x + (int64_t)d * CH;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = (c0 + g) * kWave + lane;
        if (CH % kWave == 0 || i < CH) __builtin_nontemporal_store(v[g], o + i);
      }
      if (scale_lane) __builtin_nontemporal_store(s, expand_scales + (int64_t)d * SCH + lane);
    }
    if (expand_weights != nullptr && part == 0 && lane < K && my_dst >= 0)
      expand_weights[my_dst] = topk_weights[(int64_t)t * K + lane];
  }
}

template <int ROWB, int SCB, int K>
int dispatch_impl(const DispatchArgs &a) {
  if (a.T == 0) return 0;
  constexpr int SPLIT = DispatchGeometry<ROWB / 16>::SPLIT;
  const int64_t waves = (int64_t)a.T * SPLIT;
  const int blocks = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  const bool fwd_w = a.topk_weights != nullptr && a.expand_weights != nullptr;
  ep_dispatch_expand<ROWB, SCB, K><<<blocks, kThreads, 0, a.stream>>>(
      (const u32x4 *)a.x, (const u32x4 *)a.x_scales, a.topk_weights, a.dst_slot, a.T,
      a.capacity, (u32x4 *)a.expand_x, (u32x4 *)a.expand_scales,
      fwd_w ? a.expand_weights : nullptr);
  return launch_status();
}

template <int H, int K>
int dispatch_bf16(const DispatchArgs &a) { return dispatch_impl<H * 2, 0, K>(a); }
template <int H, int K>
int dispatch_fp8(const DispatchArgs &a) { return dispatch_impl<H, (H / 128) * 4, K>(a); }

}  // namespace

#define EP_DISPATCH_K_BF16(K) \
  case K:                     \
    return dispatch_bf16<H_, K>(a);
#define EP_DISPATCH_K_FP8(K) \
  case K:                    \
    return dispatch_fp8<H_, K>(a);

template <int H_>
static int dispatch_bf16_k(const DispatchArgs &a) {
  switch (a.K) { EP_FOR_EACH_TOPK(EP_DISPATCH_K_BF16) default: return -2; }
}
template <int H_>
static int dispatch_fp8_k(const DispatchArgs &a) {
  switch (a.K) { EP_FOR_EACH_TOPK(EP_DISPATCH_K_FP8) default: return -2; }
}

#define EP_DISPATCH_H_BF16(H) \
  case H:                     \
    return dispatch_bf16_k<H>(a);
#define EP_DISPATCH_H_FP8(H) \
  case H:                    \
    return dispatch_fp8_k<H>(a);

int launch_dispatch(const DispatchArgs &a) {
  if (a.dtype == 0) {
    switch (a.H) { EP_FOR_EACH_HIDDEN_BF16(EP_DISPATCH_H_BF16) default: return -2; }
  }
  if (a.dtype == 2) {
    switch (a.H) { EP_FOR_EACH_HIDDEN_FP8(EP_DISPATCH_H_FP8) default: return -2; }
  }
  return -2;
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
  if (dtype == 0) {
    switch (H) { EP_FOR_EACH_HIDDEN_BF16(EP_IS) default: return false; }
  }
  if (dtype == 2) {
    switch (H) { EP_FOR_EACH_HIDDEN_FP8(EP_IS) default: return false; }
  }
  return false;
}

bool has_combine(int H, int K) {
  if (!has_topk(K)) return false;
  switch (H) { EP_FOR_EACH_HIDDEN_BF16(EP_IS) default: return false; }
}

}  // namespace ep
