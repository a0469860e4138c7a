// Routing layout for gfx950: per-expert counts, expert-aligned exclusive
// offsets, a destination slot per (token, k) and the receive metadata.
//
// Follows the DeepEP overall-architecture page: the EPHandle structure
// (num_unaligned_recv_tokens_perpert, psum_num_recv_tokens_per_expert with
// expert_alignment, dst_buffer_slot_idx, recv_src_metadata [num_recv, topk+2],
// num_recv_tokens, num_expanded_tokens) and the dispatch data-flow figure
// (notify warps count per expert and compute target slots). DeepEP counts
// with global atomics, which leaves the order inside an expert segment to
// chance; here every slot is a pure function of topk_idx: inside a segment
// rows go to entries in token-major (t, then k) order.
//
// Design (MI355X): entries are cut into tiles of whole tokens (up to 1024
// entries: 16, 8 or 4 wave64s of entries as E grows), one 1024-thread
// workgroup per tile, one entry per thread.
//   1. Every entry ORs its lane bit into an LDS word mask[wave][e] (the
//      result of an OR does not depend on the order of the ORs). For each
//      expert, a pass over its wave words gives the entries of that expert in
//      earlier waves; an entry's rank in the tile is that base plus the
//      popcount of its own wave word below its lane (mbcnt). The words are
//      stored wave-major, so the pass (one thread per expert) reads
//      consecutive words across lanes, free of LDS bank conflicts.
//   2. A tile's per-expert totals go to the workspace. A second launch
//      reduces, per expert, the totals of earlier tiles (prefix) and of all
//      tiles (count), pads each count to the alignment, scans over experts,
//      and writes slot = offset + prefix + rank-in-tile and the metadata.
// A single tile (small T*K) runs both halves in one launch with no
// workspace; so do up to 2^14 entries, with every block also scanning all
// entries (see ep_layout_fused_tiles). Results do not depend on scheduling.
// On request the last launch also writes the dispatch plan: each tile's
// entries in slot order, the order in which dispatch writes expand rows
// fastest (write_plan).
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "ep_device.hpp"
#include "ep_launch.hpp"

namespace ep {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesMax = kThreads / kWave;
constexpr int kRankBits = 10;  // rank inside a tile < 1024
// Largest T*K laid out by the single-launch multi-tile kernel (every block
// scans all entries); above it, two launches share per-tile histograms
// through the workspace. Measured on MI355X (E=256, top-8): one launch wins
// up to 16K entries (11.4 vs 12.8 us), two launches from 32K (12.3 vs 13.3;
// re-measured in the prefill step at 32K entries, 167.4 against 168.8 us).
constexpr int64_t kFusedMaxEntries = 1 << 14;
// Longest walk over tiles (loads per thread) the second launch of the
// many-tile path does itself; beyond it a tile-scan launch runs first.
// Measured on MI355X: without the scan 9.7 / 10.3 / 11.7 / 18.5 / 80.8 us at
// walks of 8 / 16 / 32 / 128 / 512 tiles; with it about 12-13 us, then
// growing slowly with the tile count (21 us at 512 tiles of 1024 experts).
constexpr int kScanMinWalk = 64;

// Waves of entries per tile for E experts: the lane masks (E x NW x 8 bytes)
// stay within 32 KiB of LDS.
constexpr int tile_waves(int E) { return E <= 256 ? 16 : (E <= 512 ? 8 : 4); }

template <int K, int NW>
struct Tile {
  static constexpr int tokens = NW * kWave / K;  // whole tokens per tile
  static constexpr int entries = tokens * K;     // <= NW * 64
};

struct EntryRank {
  int e;     // expert of this thread's entry, -1 if masked or absent
  int rank;  // entries of the same expert earlier in the tile
};

__host__ __device__ constexpr size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

// LDS of the rank phase: lane masks [E][NW], per-wave bases [E][NW], tile
// totals [E], token flags [kThreads].
__host__ __device__ constexpr size_t rank_lds_bytes(int E, int NW) {
  return align16((size_t)E * NW * 8) + align16((size_t)E * NW * 2) + align16((size_t)E * 4) +
         (size_t)kThreads * 4;
}

extern __shared__ __align__(16) unsigned char g_smem[];

struct RankLds {
  uint64_t *mask;
  uint16_t *wbase;
  int *total;
  int *tok;
};

__device__ __forceinline__ RankLds rank_lds(int E, int NW) {
  unsigned char *p = g_smem;
  RankLds s;
  s.mask = (uint64_t *)p;
  p += align16((size_t)E * NW * 8);
  s.wbase = (uint16_t *)p;
  p += align16((size_t)E * NW * 2);
  s.total = (int *)p;
  p += align16((size_t)E * 4);
  s.tok = (int *)p;
  return s;
}

// Optional read-ahead of memory the caller reads next (the token rows, before
// dispatch). The layout's launches leave most of the chip idle; workgroups
// added after the layout's own read one 4-byte word of every 128-byte line of
// their share with ordinary loads, which pulls those lines into the
// last-level cache while the layout runs. The words are only kept alive, never
// used. Measured on MI355X (prefill, 58.7 MB of rows evicted from the cache):
// with the rows read ahead, dispatch takes about as long as with the rows
// cached (a burst of reads while the layout runs costs far less than the same
// reads interleaved with dispatch's writes).
struct Prefetch {
  const uint32_t *p;  // NULL: none
  int64_t l0, l1;     // this launch's share, in 128-byte lines from p
  int blocks;         // workgroups given to it, after the layout's own
};

__device__ __forceinline__ void prefetch_share(const Prefetch &pf, int q) {
  constexpr int kDepth = 8;  // loads in flight per lane
  const int lane = lane_id();
  const int64_t w = (int64_t)q * kWavesMax + threadIdx.x / kWave;
  const int64_t nw = (int64_t)pf.blocks * kWavesMax;
  // groups of 64 lines, one per load instruction: wave w takes groups w, w + nw, ...
  const int64_t groups = (pf.l1 - pf.l0 + kWave - 1) / kWave;
  for (int64_t g0 = w; g0 < groups; g0 += nw * kDepth) {
    uint32_t v[kDepth];
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
      const int64_t l = pf.l0 + (g0 + j * nw) * kWave + lane;
      v[j] = l < pf.l1 ? pf.p[l * 32] : 0u;
    }
#pragma unroll
    for (int j = 0; j < kDepth; ++j) asm volatile("" ::"v"(v[j]));
  }
}

// Step 1. Also leaves s.tok[j] = 1 for every token j of the tile with an
// unmasked entry (0 otherwise) and s.total[e] = entries of expert e.
template <int K, int NW>
__device__ EntryRank tile_rank(const int32_t *__restrict__ topk_idx, int64_t t0, int ntok, int E,
                               const RankLds &s) {
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  // the id load is issued first, so that its latency overlaps the LDS clearing
  const int v = tid < ntok * K ? topk_idx[t0 * K + tid] : -1;
  for (int i = tid; i < E * NW; i += kThreads) s.mask[i] = 0;
  if (tid < Tile<K, NW>::tokens) s.tok[tid] = 0;
  const int e = (v >= 0 && v < E) ? v : -1;
  __syncthreads();
  if (e >= 0) {
    __hip_atomic_fetch_or(&s.mask[w * E + e], 1ull << lane, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WORKGROUP);
    s.tok[tid / K] = 1;  // every writer stores the same value
  }
  __syncthreads();
  for (int ex = tid; ex < E; ex += kThreads) {
    uint64_t m[NW];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) m[ww] = s.mask[ww * E + ex];
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      s.wbase[ww * E + ex] = (uint16_t)run;
      run += __popcll(m[ww]);
    }
    s.total[ex] = run;
  }
  __syncthreads();
  int rank = 0;
  if (e >= 0) rank = s.wbase[w * E + e] + count_below(s.mask[w * E + e]);
  return {e, rank};
}

// Block-wide reductions split around a barrier that the caller places, so
// that several of them, and other LDS writes, share one barrier. Each
// *_publish writes one int per wave into its own LDS array (kWavesMax ints);
// after the barrier the matching *_collect reads all of them. Such an array
// is not written again until every thread has passed a later barrier.

// Sum over the block: the wave's sum of v.
__device__ __forceinline__ void sum_publish(int v, int *s_w) {
  v = wave_sum(v);
  if (lane_id() == 0) s_w[threadIdx.x / kWave] = v;
}
__device__ __forceinline__ int sum_collect(const int *s_w) {
  int t = 0;
#pragma unroll
  for (int ww = 0; ww < kWavesMax; ++ww) t += s_w[ww];
  return t;
}

// Exclusive prefix of v over the block in thread order: publish returns the
// inclusive prefix within the wave; collect adds the totals of earlier waves
// and gives the block total.
__device__ __forceinline__ int scan_publish(int v, int *s_w) {
  const int inc = wave_inclusive_scan(v);
  if (lane_id() == kWave - 1) s_w[threadIdx.x / kWave] = inc;
  return inc;
}
__device__ __forceinline__ int scan_collect(int inc, int v, const int *s_w, int &total) {
  const int w = threadIdx.x / kWave;
  int before = 0, t = 0;
#pragma unroll
  for (int ww = 0; ww < kWavesMax; ++ww) {
    const int x = s_w[ww];
    before += ww < w ? x : 0;
    t += x;
  }
  total = t;
  return before + inc - v;
}

// Rank of a set flag among the block's set flags (those of lower threads);
// collect also gives the block's count.
__device__ __forceinline__ uint64_t flag_publish(bool f, int *s_w) {
  const uint64_t bits = ballot(f);
  if (lane_id() == 0) s_w[threadIdx.x / kWave] = __popcll(bits);
  return bits;
}
__device__ __forceinline__ int flag_collect(uint64_t bits, const int *s_w, int &total) {
  const int w = threadIdx.x / kWave;
  int before = 0, t = 0;
#pragma unroll
  for (int ww = 0; ww < kWavesMax; ++ww) {
    const int c = s_w[ww];
    before += ww < w ? c : 0;
    t += c;
  }
  total = t;
  return before + count_below(bits);
}

// Writes the tile's final slots and metadata rows. s_row[j] must hold the
// receive row of token j of the tile, or -1.
template <int K>
__device__ __forceinline__ void write_slots_and_meta(int64_t t0, int ntok, int slot,
                                                     const int *s_row,
                                                     int32_t *__restrict__ dst_slot,
                                                     int32_t *__restrict__ meta) {
  const int tid = threadIdx.x;
  if (tid < ntok * K) {
    dst_slot[t0 * K + tid] = slot;
    const int j = tid / K, k = tid - j * K;
    const int row = s_row[j];
    if (row >= 0) {
      int32_t *m = meta + (int64_t)row * (K + 2);
      m[2 + k] = slot;
      if (k == 0) {
        m[0] = (int32_t)(t0 + j);
        m[1] = 0;  // source rank: a world of one
      }
    }
  }
}

// Writes the tile's part of the dispatch plan: the tile's unmasked entries in
// ascending slot order, each as (entry t*K + k, slot), then (-1, -1) for its
// masked entries. Inside a tile, slots ascend with (expert, rank), so an
// entry's place is the count of the tile's entries of lower experts (s_tb,
// an exclusive scan over experts of the tile's counts, published by a
// barrier) plus its rank; nvalid is the tile's count of unmasked entries.
template <int K>
__device__ __forceinline__ void write_plan(int64_t t0, int ntok, int e, int rank, int slot,
                                           const int *s_tb, int nvalid,
                                           int32_t *__restrict__ plan) {
  const int tid = threadIdx.x;
  if (tid < ntok * K) {
    int2 *p = reinterpret_cast<int2 *>(plan) + t0 * K;
    if (e >= 0) p[s_tb[e] + rank] = make_int2((int)(t0 * K) + tid, slot);
    if (tid >= nvalid) p[tid] = make_int2(-1, -1);
  }
}

// One launch for T*K that fits a single tile (including T = 0).
template <int K, int NW>
__global__ __launch_bounds__(kThreads) void ep_layout_single_tile(
    const int32_t *__restrict__ topk_idx, int T, int E, int A, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv, int32_t *__restrict__ plan, Prefetch pf) {
  if (blockIdx.x >= 1) {  // read-ahead workgroups
    prefetch_share(pf, blockIdx.x - 1);
    return;
  }
  __shared__ int s_scan[2 * kWavesMax];
  __shared__ int s_flag[kWavesMax];
  const RankLds s = rank_lds(E, NW);
  int *s_off = (int *)(g_smem + rank_lds_bytes(E, NW));  // E
  int *s_tb = s_off + E;                                 // E: dispatch plan
  const int tid = threadIdx.x;

  const EntryRank r = tile_rank<K, NW>(topk_idx, 0, T, E, s);
  const int cnt = tid < E ? s.total[tid] : 0;
  const int padded = ((cnt + A - 1) / A) * A;
  const int inc_off = scan_publish(padded, s_scan);
  const int inc_tb = scan_publish(cnt, s_scan + kWavesMax);
  const bool f = tid < T && s.tok[tid] != 0;  // only thread tid reads or writes s.tok[tid] here
  const uint64_t fbits = flag_publish(f, s_flag);
  __syncthreads();
  int rows, nvalid, nrecv;
  const int off = scan_collect(inc_off, padded, s_scan, rows);
  const int tb = scan_collect(inc_tb, cnt, s_scan + kWavesMax, nvalid);
  const int tok_rank = flag_collect(fbits, s_flag, nrecv);
  if (tid < E) {
    s_off[tid] = off;
    s_tb[tid] = tb;
    counts[tid] = cnt;
    offsets[tid] = off;
  }
  if (tid == 0) {
    offsets[E] = rows;
    *num_recv = nrecv;
  }
  if (tid < T) s.tok[tid] = f ? tok_rank : -1;
  __syncthreads();  // publishes s_off, s_tb and the receive rows
  const int slot = r.e >= 0 ? s_off[r.e] + r.rank : -1;
  write_slots_and_meta<K>(0, T, slot, s.tok, dst_slot, meta);
  if (plan != nullptr) write_plan<K>(0, T, r.e, r.rank, slot, s_tb, nvalid, plan);
}

// Copies one (entry j, 1 KiB slice) unit of the fused layout + dispatch
// launch to expand row d; slice 0 also carries the scale row and the weight.
// v is the lane's chunk of the row slice, already loaded.
template <bool WIDE>
__device__ __forceinline__ void copy_unit(const u32x4 &v, int64_t t, int j, int slice, int d,
                                          int row_chunks, const u32x4 *__restrict__ x_scales,
                                          int scale_chunks, const float *__restrict__ topk_weights,
                                          u32x4 *__restrict__ expand_x,
                                          u32x4 *__restrict__ expand_scales,
                                          float *__restrict__ expand_weights) {
  const int lane = lane_id();
  const int c = slice * kWave + lane;
  if (c < row_chunks)
    store_row<WIDE ? RowStore::kNtDevice : RowStore::kNt>(
        v, expand_x + (int64_t)d * row_chunks, row_chunks * 16, c * 16);
  if (slice == 0) {
    if (x_scales != nullptr)
      for (int q = lane; q < scale_chunks; q += kWave)
        __builtin_nontemporal_store(x_scales[t * scale_chunks + q],
                                    expand_scales + (int64_t)d * scale_chunks + q);
    if (expand_weights != nullptr && lane == 0) expand_weights[d] = topk_weights[j];
  }
}

// Rank of copy workgroup g among the n workgroups first .. first+n-1 of a
// launch once they are grouped by XCD: the dispatcher deals workgroups to the
// 8 XCDs in turn, so workgroups whose offsets from `first` agree modulo 8 share
// an XCD and its L2, and each such group gets a contiguous range of ranks (a
// bijection onto [0, n) for any n). Consecutive copy units then run on one XCD,
// so the K entries of a token read its x slices through one L2 instead of up
// to K of them.
constexpr int kXcdCount = 8;
__device__ __forceinline__ int xcd_rank(int g, int first, int n) {
  const int b = g - first, y = b % kXcdCount, q = n / kXcdCount, r = n % kXcdCount;
  return y * q + (y < r ? y : r) + b / kXcdCount;
}

// The copy workgroups of the fused launch when expert_alignment is 1
// (COUNTED): no ranking at all. Without alignment padding an entry's slot is
// the number of unmasked entries whose key (expert id, entry index) is
// smaller than its own: the entries of lower experts (the expert's offset)
// plus the earlier entries of its own expert (its rank). The workgroup
// stages the T*K keys in LDS once (a masked entry gets the largest key);
// each lane then holds 16 of them, and a wave counts, for each entry it
// copies, the keys below that entry's key and sums the count over the wave.
// The row slices of a wave's first kPre units are loaded before the keys are
// staged, so their latencies overlap each other and the key load. Workgroup
// 0 writes the layout's outputs and copies nothing; workgroups 1.. share the
// (entry, slice) units.
template <int K, bool WIDE>
__device__ __forceinline__ void copy_counted(
    const int32_t *__restrict__ topk_idx, int T, int E, const u32x4 *__restrict__ x,
    int row_chunks, const u32x4 *__restrict__ x_scales, int scale_chunks,
    const float *__restrict__ topk_weights, int64_t capacity, u32x4 *__restrict__ expand_x,
    u32x4 *__restrict__ expand_scales, float *__restrict__ expand_weights, FastDiv by_slices) {
  constexpr int kNoKey = 0x7fffffff;
  constexpr int kPre = 4;  // units per wave whose row slices load before the keys
  int *s_key = (int *)g_smem;  // kThreads keys
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int n = T * K;  // <= kThreads (one tile)
  const int slices = (row_chunks + kWave - 1) / kWave;
  // 32-bit unit indices (n * slices < 2^20) and a multiply-shift division by
  // the slice count: the index arithmetic sits on each wave's path to its
  // first load.
  const int units = n * slices;
  const int ncopy = (int)gridDim.x - 1;
  const int stride = ncopy * kWavesMax;
  const int u0 = xcd_rank((int)blockIdx.x, 1, ncopy) * kWavesMax + wave;
  auto load = [&](int u) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (u < units) {
      const int j = (int)fast_div_apply((uint32_t)u, by_slices);
      const int c = (u - j * slices) * kWave + lane;
      if (c < row_chunks) v = x[(int64_t)(j / K) * row_chunks + c];
    }
    return v;
  };
  u32x4 pre[kPre];
#pragma unroll
  for (int p = 0; p < kPre; ++p) pre[p] = load(u0 + p * stride);
  const int id = tid < n ? topk_idx[tid] : -1;
  s_key[tid] = (id >= 0 && id < E) ? (id << kRankBits) | tid : kNoKey;
  __syncthreads();
  int key[kWavesMax];  // entries q * 64 + lane
#pragma unroll
  for (int q = 0; q < kWavesMax; ++q) key[q] = s_key[q * kWave + lane];
  auto copy = [&](int u, const u32x4 &v) {
    const int j = (int)fast_div_apply((uint32_t)u, by_slices);
    const int slice = u - j * slices;
    const int kj = __builtin_amdgcn_readfirstlane(s_key[j]);
    if (kj == kNoKey) return;  // masked: no slot
    int below = 0;
#pragma unroll
    for (int q = 0; q < kWavesMax; ++q) below += key[q] < kj ? 1 : 0;
    const int d = __builtin_amdgcn_readfirstlane(wave_sum(below));
    if (d >= capacity) return;
    copy_unit<WIDE>(v, j / K, j, slice, d, row_chunks, x_scales, scale_chunks, topk_weights,
                    expand_x, expand_scales, expand_weights);
  };
#pragma unroll
  for (int p = 0; p < kPre; ++p)
    if (u0 + p * stride < units) copy(u0 + p * stride, pre[p]);
  for (int u = u0 + kPre * stride; u < units; u += stride) copy(u, load(u));
}

// Layout and dispatch in one launch for a batch that fits one tile (a
// decode step, say), after the dispatch kernels of the DeepEP page, whose
// notify warps compute the slots inside dispatch. Every workgroup ranks all
// entries in its own LDS exactly as ep_layout_single_tile does, and
// workgroup 0 also writes the layout's outputs. Each workgroup then copies
// its share of (entry, 1 KiB slice) units token-major, with the slots read
// from its own LDS. The ranking is repeated per workgroup, a few microseconds
// of LDS work in parallel. That costs less than a second launch and the
// round trip of dst_slot through memory. COUNTED (expert_alignment 1,
// uncapped): only workgroup 0 ranks, to write the layout's outputs, and the
// other workgroups find their entries' slots by counting keys
// (copy_counted). Row and scale-row widths are run-time values (16-byte
// chunks). WIDE: launched uncapped, which selects the device-scope
// non-temporal row store, as ep_dispatch_expand uses.
template <int K, int NW, bool WIDE, bool COUNTED>
__global__ __launch_bounds__(kThreads) void ep_layout_dispatch_tile(
    const int32_t *__restrict__ topk_idx, int T, int E, int A, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv, const u32x4 *__restrict__ x, int row_chunks,
    const u32x4 *__restrict__ x_scales, int scale_chunks, const float *__restrict__ topk_weights,
    int64_t capacity, u32x4 *__restrict__ expand_x, u32x4 *__restrict__ expand_scales,
    float *__restrict__ expand_weights, FastDiv by_slices) {
  if (COUNTED && blockIdx.x != 0) {
    copy_counted<K, WIDE>(topk_idx, T, E, x, row_chunks, x_scales, scale_chunks, topk_weights,
                          capacity, expand_x, expand_scales, expand_weights, by_slices);
    return;
  }
  __shared__ int s_scan[kWavesMax];
  __shared__ int s_flag[kWavesMax];
  const RankLds s = rank_lds(E, NW);
  int *s_off = (int *)(g_smem + rank_lds_bytes(E, NW));  // E
  int *s_slot = s_off + E;                               // kThreads: slot of entry tid
  const int tid = threadIdx.x;

  const EntryRank r = tile_rank<K, NW>(topk_idx, 0, T, E, s);
  const int cnt = tid < E ? s.total[tid] : 0;
  const int padded = ((cnt + A - 1) / A) * A;
  const int inc_off = scan_publish(padded, s_scan);
  const bool f = tid < T && s.tok[tid] != 0;  // only thread tid reads or writes s.tok[tid] here
  const uint64_t fbits = flag_publish(f, s_flag);
  __syncthreads();
  int rows, nrecv;
  const int off = scan_collect(inc_off, padded, s_scan, rows);
  const int tok_rank = flag_collect(fbits, s_flag, nrecv);
  if (tid < E) s_off[tid] = off;
  if (blockIdx.x == 0) {  // the layout's outputs, as ep_layout_single_tile writes them
    if (tid < E) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == 0) {
      offsets[E] = rows;
      *num_recv = nrecv;
    }
    if (tid < T) s.tok[tid] = f ? tok_rank : -1;
  }
  __syncthreads();  // publishes s_off (and in workgroup 0 the receive rows)
  const int slot = r.e >= 0 ? s_off[r.e] + r.rank : -1;
  if (blockIdx.x == 0) write_slots_and_meta<K>(0, T, slot, s.tok, dst_slot, meta);
  if (COUNTED) return;  // workgroup 0 copies nothing
  s_slot[tid] = slot;
  __syncthreads();  // publishes s_slot

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int slices = (row_chunks + kWave - 1) / kWave;
  const int units = T * K * slices;  // one tile: below 2^20
  const int stride = (int)gridDim.x * kWavesMax;
  const int u0 = xcd_rank((int)blockIdx.x, 0, (int)gridDim.x) * kWavesMax + wave;
  for (int u = u0; u < units; u += stride) {
    const int j = (int)fast_div_apply((uint32_t)u, by_slices);  // entry t*K + k
    const int slice = u - j * slices;
    const int d = __builtin_amdgcn_readfirstlane(s_slot[j]);
    if (d < 0 || d >= capacity) continue;
    const int64_t t = j / K;
    const int c = slice * kWave + lane;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < row_chunks) v = x[t * row_chunks + c];
    copy_unit<WIDE>(v, t, j, slice, d, row_chunks, x_scales, scale_chunks, topk_weights,
                    expand_x, expand_scales, expand_weights);
  }
}

// Layout and non-expand dispatch in one launch for a batch that fits one
// tile, as ep_layout_dispatch_tile does for the expand buffer: every
// workgroup ranks the entries and the received tokens in its own LDS and
// workgroup 0 writes the layout's outputs; then each workgroup copies its
// share of (token, 1 KiB slice) units of the received tokens to their
// receive rows, with the rows, ids and weights ep_dispatch_compact writes
// (an entry has a slot exactly when its id lies in [0, E)). WIDE: launched
// uncapped, which keeps the received rows at device scope, as
// ep_dispatch_compact does.
template <int K, int NW, bool WIDE>
__global__ __launch_bounds__(kThreads) void ep_layout_dispatch_compact_tile(
    const int32_t *__restrict__ topk_idx, int T, int E, int A, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv, const u32x4 *__restrict__ x, int row_chunks,
    const float *__restrict__ x_scales, int scale_cols, const float *__restrict__ topk_weights,
    u32x4 *__restrict__ recv_x, float *__restrict__ recv_scales,
    int32_t *__restrict__ recv_topk_idx, float *__restrict__ recv_topk_weights,
    FastDiv by_slices) {
  __shared__ int s_scan[kWavesMax];
  __shared__ int s_flag[kWavesMax];
  const RankLds s = rank_lds(E, NW);
  int *s_off = (int *)(g_smem + rank_lds_bytes(E, NW));  // E
  const int tid = threadIdx.x;

  const EntryRank r = tile_rank<K, NW>(topk_idx, 0, T, E, s);
  const int cnt = tid < E ? s.total[tid] : 0;
  const int padded = ((cnt + A - 1) / A) * A;
  const int inc_off = scan_publish(padded, s_scan);
  const bool f = tid < T && s.tok[tid] != 0;  // only thread tid reads or writes s.tok[tid] here
  const uint64_t fbits = flag_publish(f, s_flag);
  __syncthreads();
  int rows, nrecv;
  const int off = scan_collect(inc_off, padded, s_scan, rows);
  const int tok_rank = flag_collect(fbits, s_flag, nrecv);
  if (tid < T) s.tok[tid] = f ? tok_rank : -1;
  if (blockIdx.x == 0) {  // the layout's outputs, as ep_layout_single_tile writes them
    if (tid < E) {
      s_off[tid] = off;
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == 0) {
      offsets[E] = rows;
      *num_recv = nrecv;
    }
  }
  __syncthreads();  // publishes the receive rows (and in workgroup 0 s_off)
  if (blockIdx.x == 0)
    write_slots_and_meta<K>(0, T, r.e >= 0 ? s_off[r.e] + r.rank : -1, s.tok, dst_slot, meta);

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int slices = (row_chunks + kWave - 1) / kWave;
  const int units = T * slices;  // one tile: below 2^20
  const int stride = (int)gridDim.x * kWavesMax;
  for (int u = (int)blockIdx.x * kWavesMax + wave; u < units; u += stride) {
    const int t = (int)fast_div_apply((uint32_t)u, by_slices);
    const int slice = u - t * slices;
    const int i = __builtin_amdgcn_readfirstlane(s.tok[t]);  // receive row, or -1
    if (i < 0) continue;
    const int c = slice * kWave + lane;
    if (c < row_chunks)
      store_row<WIDE ? RowStore::kDevice : RowStore::kNt>(
          x[(int64_t)t * row_chunks + c], recv_x + (int64_t)i * row_chunks, row_chunks * 16,
          c * 16);
    if (slice == 0) {
      if (recv_scales != nullptr)
        for (int j = lane; j < scale_cols; j += kWave)
          recv_scales[(int64_t)i * scale_cols + j] = x_scales[(int64_t)t * scale_cols + j];
      for (int k = lane; k < K; k += kWave) {
        const int64_t tk = (int64_t)t * K + k;
        const int id = topk_idx[tk];
        recv_topk_idx[(int64_t)i * K + k] = id >= 0 && id < E ? id : -1;
        if (recv_topk_weights != nullptr) recv_topk_weights[(int64_t)i * K + k] = topk_weights[tk];
      }
    }
  }
}

// One launch for several tiles when T*K is small enough: besides ranking its
// own tile, every block streams all of topk_idx (from L2) into LDS integer
// histograms of the entries before its tile and of all entries, and counts
// received tokens the same way. Integer sums do not depend on the order of
// the atomic adds, so the result is still a pure function of topk_idx. The
// redundant scan costs O(T*K) per block, which is why larger inputs take the
// two-launch path instead.
template <int K, int NW>
__device__ __forceinline__ void fused_tile(
    const int32_t *__restrict__ topk_idx, int T, int E, int A, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv, int32_t *__restrict__ plan, const int b) {
  __shared__ int s_sum[2 * kWavesMax];
  __shared__ int s_scan[2 * kWavesMax];
  __shared__ int s_flag[kWavesMax];
  const RankLds s = rank_lds(E, NW);
  int *s_pre = (int *)(g_smem + rank_lds_bytes(E, NW));  // E: entries before this tile
  int *s_all = s_pre + E;                                // E: all entries
  int *s_off = s_all + E;                                // E
  int *s_tb = s_off + E;                                 // E: dispatch plan
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)b * Tile<K, NW>::tokens;
  const int ntok = (int)min((int64_t)Tile<K, NW>::tokens, (int64_t)T - t0);

  for (int ex = tid; ex < E; ex += kThreads) {
    s_pre[ex] = 0;
    s_all[ex] = 0;
  }
  // Barriers inside tile_rank order the zeroing above before the adds below.
  const EntryRank r = tile_rank<K, NW>(topk_idx, t0, ntok, E, s);
  int vpre = 0, vall = 0;
  for (int64_t j = tid; j < T; j += kThreads) {  // token-major: coalesced rows of K ids
    int ids[K];
#pragma unroll
    for (int k = 0; k < K; ++k) ids[k] = topk_idx[j * K + k];
    const bool before = j < t0;
    bool any = false;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int e = ids[k];
      if (e >= 0 && e < E) {
        any = true;
        __hip_atomic_fetch_add(&s_all[e], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (before)
          __hip_atomic_fetch_add(&s_pre[e], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    vall += any ? 1 : 0;
    vpre += (any && before) ? 1 : 0;
  }
  sum_publish(vpre, s_sum);
  sum_publish(vall, s_sum + kWavesMax);
  const bool f = tid < ntok && s.tok[tid] != 0;  // only thread tid reads or writes s.tok[tid] here
  const uint64_t fbits = flag_publish(f, s_flag);
  __syncthreads();  // publishes the histograms, the wave sums and the flag counts
  const int recv_before = sum_collect(s_sum);
  const int recv_total = sum_collect(s_sum + kWavesMax);
  int nflag;
  const int tok_rank = flag_collect(fbits, s_flag, nflag);
  const int cnt = tid < E ? s_all[tid] : 0;
  const int padded = ((cnt + A - 1) / A) * A;
  const int mine = tid < E ? s.total[tid] : 0;  // this tile's count of expert tid
  const int inc_off = scan_publish(padded, s_scan);
  const int inc_tb = scan_publish(mine, s_scan + kWavesMax);
  if (tid < ntok) s.tok[tid] = f ? recv_before + tok_rank : -1;
  __syncthreads();
  int rows, nvalid;
  const int off = scan_collect(inc_off, padded, s_scan, rows);
  const int tb = scan_collect(inc_tb, mine, s_scan + kWavesMax, nvalid);
  if (tid < E) {
    s_off[tid] = off;
    s_tb[tid] = tb;
  }
  if (b == 0) {
    if (tid < E) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == 0) {
      offsets[E] = rows;
      *num_recv = recv_total;
    }
  }
  __syncthreads();  // publishes s_off and s_tb
  const int slot = r.e >= 0 ? s_off[r.e] + s_pre[r.e] + r.rank : -1;
  write_slots_and_meta<K>(t0, ntok, slot, s.tok, dst_slot, meta);
  if (plan != nullptr) write_plan<K>(t0, ntok, r.e, r.rank, slot, s_tb, nvalid, plan);
}

// Tile blockIdx.x, or with LOOP (the stream caps the workgroup count below
// the tile count) tiles blockIdx.x, blockIdx.x + gridDim.x, ...; the barrier
// lets the next tile reuse LDS. Without LOOP there is no loop to keep values
// live across, which saves registers and a microsecond.
template <int K, int NW, bool LOOP>
__global__ __launch_bounds__(kThreads) void ep_layout_fused_tiles(
    const int32_t *__restrict__ topk_idx, int T, int E, int A, int num_tiles,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot,
    int32_t *__restrict__ meta, int32_t *__restrict__ num_recv, int32_t *__restrict__ plan,
    Prefetch pf) {
  if constexpr (!LOOP) {
    if ((int)blockIdx.x >= num_tiles) {  // read-ahead workgroups
      prefetch_share(pf, blockIdx.x - num_tiles);
      return;
    }
    fused_tile<K, NW>(topk_idx, T, E, A, counts, offsets, dst_slot, meta, num_recv, plan,
                      blockIdx.x);
  } else {
    for (int b = blockIdx.x; b < num_tiles; b += gridDim.x) {
      fused_tile<K, NW>(topk_idx, T, E, A, counts, offsets, dst_slot, meta, num_recv, plan, b);
      __syncthreads();
    }
  }
}

// First launch of the multi-tile path: per-tile histograms and ranks.
// dst_slot temporarily holds (expert << kRankBits | rank-in-tile), or -1.
template <int K, int NW>
__device__ __forceinline__ void histogram_tile(
    const int32_t *__restrict__ topk_idx, int T, int E, int32_t *__restrict__ dst_slot,
    int32_t *__restrict__ tile_counts, int32_t *__restrict__ tile_recv, const int b) {
  __shared__ int s_flag[kWavesMax];
  const RankLds s = rank_lds(E, NW);
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)b * Tile<K, NW>::tokens;
  const int ntok = (int)min((int64_t)Tile<K, NW>::tokens, (int64_t)T - t0);

  const EntryRank r = tile_rank<K, NW>(topk_idx, t0, ntok, E, s);
  if (tid < ntok * K) dst_slot[t0 * K + tid] = r.e >= 0 ? (r.e << kRankBits) | r.rank : -1;
  for (int ex = tid; ex < E; ex += kThreads) tile_counts[(int64_t)b * E + ex] = s.total[ex];
  flag_publish(tid < ntok && s.tok[tid] != 0, s_flag);
  __syncthreads();
  if (tid == 0) tile_recv[b] = sum_collect(s_flag);
}

template <int K, int NW, bool LOOP>
__global__ __launch_bounds__(kThreads) void ep_layout_tile_histogram(
    const int32_t *__restrict__ topk_idx, int T, int E, int num_tiles,
    int32_t *__restrict__ dst_slot, int32_t *__restrict__ tile_counts,
    int32_t *__restrict__ tile_recv, Prefetch pf) {
  if constexpr (!LOOP) {
    if ((int)blockIdx.x >= num_tiles) {  // read-ahead workgroups
      prefetch_share(pf, blockIdx.x - num_tiles);
      return;
    }
    histogram_tile<K, NW>(topk_idx, T, E, dst_slot, tile_counts, tile_recv, blockIdx.x);
  } else {
    for (int b = blockIdx.x; b < num_tiles; b += gridDim.x) {
      histogram_tile<K, NW>(topk_idx, T, E, dst_slot, tile_counts, tile_recv, b);
      __syncthreads();
    }
  }
}

// Per-tile prefixes computed by ep_layout_tile_scan (used when there are
// many tiles): exclusive prefix over tiles of each expert's count, the
// expert totals, and the same for received tokens.
struct TileScan {
  const int32_t *tile_base;     // [B][E]
  const int32_t *expert_total;  // [E]
  const int32_t *recv_base;     // [B]
  const int32_t *recv_total;    // [1]
};

// Second launch: offsets, final slots and metadata for tile b. Without
// SCANNED every block sums the per-tile counts of all tiles itself (P threads
// per expert); with SCANNED it reads the prefixes of ep_layout_tile_scan.
template <int K, int NW, bool SCANNED>
__device__ __forceinline__ void assign_tile(
    int T, int E, int A, int num_tiles, const int32_t *__restrict__ tile_counts,
    const int32_t *__restrict__ tile_recv, const TileScan &scan, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv, int32_t *__restrict__ plan, const int b) {
  __shared__ int s_pre[kThreads];
  __shared__ int s_tot[kThreads];
  __shared__ int s_row[kThreads];
  __shared__ int s_sum[2 * kWavesMax];
  __shared__ int s_scan[2 * kWavesMax];
  __shared__ int s_flag[kWavesMax];
  int *s_base = (int *)g_smem;  // E
  int *s_off = s_base + E;      // E
  int *s_tb = s_off + E;        // E: dispatch plan
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)b * Tile<K, NW>::tokens;
  const int ntok = (int)min((int64_t)Tile<K, NW>::tokens, (int64_t)T - t0);

  // Every global load of the block is issued before the first barrier.
  const int packed = tid < ntok * K ? dst_slot[t0 * K + tid] : -1;
  const int mine = plan != nullptr && tid < E ? tile_counts[(int64_t)b * E + tid] : 0;
  // P threads share an expert when the block sums the tile counts itself.
  const int epad = E <= 1 ? 1 : 1 << (32 - __builtin_clz((unsigned)(E - 1)));
  const int P = kThreads / epad;
  int base = 0, cnt = 0, recv_before = 0, recv_total = 0;
  if constexpr (SCANNED) {
    if (tid < E) {
      base = scan.tile_base[(int64_t)b * E + tid];
      cnt = scan.expert_total[tid];
    }
    recv_before = scan.recv_base[b];
    recv_total = *scan.recv_total;
  } else {
    // Per expert: entries in tiles before b, and in all tiles. P threads share
    // an expert so that each thread has only a few loads, all in flight.
    const int ex = tid % epad, part = tid / epad;
    int pre = 0, tot = 0;
    if (ex < E) {
#pragma unroll 8
      for (int bb = part; bb < num_tiles; bb += P) {
        const int c = tile_counts[(int64_t)bb * E + ex];
        tot += c;
        pre += bb < b ? c : 0;
      }
    }
    int vpre = 0, vtot = 0;
    for (int bb = tid; bb < num_tiles; bb += kThreads) {
      const int c = tile_recv[bb];
      vtot += c;
      vpre += bb < b ? c : 0;
    }
    s_pre[tid] = pre;
    s_tot[tid] = tot;
    sum_publish(vpre, s_sum);
    sum_publish(vtot, s_sum + kWavesMax);
  }
  if (tid < Tile<K, NW>::tokens) s_row[tid] = 0;
  __syncthreads();  // publishes the partial sums and the cleared token flags
  if constexpr (!SCANNED) {
    recv_before = sum_collect(s_sum);
    recv_total = sum_collect(s_sum + kWavesMax);
    if (tid < E) {
      for (int j = 0; j < P; ++j) {
        base += s_pre[j * epad + tid];
        cnt += s_tot[j * epad + tid];
      }
    }
  }
  if (packed >= 0) s_row[tid / K] = 1;  // every writer stores the same value
  const int padded = ((cnt + A - 1) / A) * A;
  const int inc_off = scan_publish(padded, s_scan);
  const int inc_tb = scan_publish(mine, s_scan + kWavesMax);
  __syncthreads();  // publishes the wave scans and the token flags
  int rows, nvalid;
  const int off = scan_collect(inc_off, padded, s_scan, rows);
  const int tb = scan_collect(inc_tb, mine, s_scan + kWavesMax, nvalid);
  if (tid < E) {
    s_base[tid] = base;
    s_off[tid] = off;
    s_tb[tid] = tb;
  }
  if (b == 0) {
    if (tid < E) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == 0) {
      offsets[E] = rows;
      *num_recv = recv_total;
    }
  }
  const bool f = tid < ntok && s_row[tid] != 0;  // only thread tid reads or writes s_row[tid] now
  const uint64_t fbits = flag_publish(f, s_flag);
  __syncthreads();  // publishes s_base, s_off, s_tb and the flag counts
  int nflag;
  const int tok_rank = flag_collect(fbits, s_flag, nflag);
  int slot = -1;
  if (packed >= 0) {
    const int e = packed >> kRankBits;
    slot = s_off[e] + s_base[e] + (packed & ((1 << kRankBits) - 1));
  }
  if (tid < ntok) s_row[tid] = f ? recv_before + tok_rank : -1;
  __syncthreads();  // publishes the receive rows
  write_slots_and_meta<K>(t0, ntok, slot, s_row, dst_slot, meta);
  if (plan != nullptr) {
    const int e = packed >= 0 ? packed >> kRankBits : -1;
    const int rank = packed & ((1 << kRankBits) - 1);
    write_plan<K>(t0, ntok, e, rank, slot, s_tb, nvalid, plan);
  }
}

template <int K, int NW, bool LOOP, bool SCANNED>
__global__ __launch_bounds__(kThreads) void ep_layout_tile_assign(
    int T, int E, int A, int num_tiles, const int32_t *__restrict__ tile_counts,
    const int32_t *__restrict__ tile_recv, TileScan scan, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv, int32_t *__restrict__ plan, Prefetch pf) {
  if constexpr (!LOOP) {
    if ((int)blockIdx.x >= num_tiles) {  // read-ahead workgroups
      prefetch_share(pf, blockIdx.x - num_tiles);
      return;
    }
    assign_tile<K, NW, SCANNED>(T, E, A, num_tiles, tile_counts, tile_recv, scan, counts, offsets,
                                dst_slot, meta, num_recv, plan, blockIdx.x);
  } else {
    for (int b = blockIdx.x; b < num_tiles; b += gridDim.x) {
      assign_tile<K, NW, SCANNED>(T, E, A, num_tiles, tile_counts, tile_recv, scan, counts,
                                  offsets, dst_slot, meta, num_recv, plan, b);
      __syncthreads();
    }
  }
}

// Middle launch of the many-tile path: for every expert e (one lane each, 64
// experts per block; column E stands for the received-token counts), the
// exclusive prefix over tiles of its per-tile count and its total. The 16
// waves of a block split the tiles into 16 runs; each lane loads a batch of
// its run's values before summing them, so a batch costs one load latency.
constexpr int kScanBatch = 16;
__global__ __launch_bounds__(kThreads) void ep_layout_tile_scan(
    const int32_t *__restrict__ tile_counts, const int32_t *__restrict__ tile_recv, int B, int E,
    int32_t *__restrict__ tile_base, int32_t *__restrict__ expert_total,
    int32_t *__restrict__ recv_base, int32_t *__restrict__ recv_total) {
  __shared__ int s_part[kWavesMax][kWave];
  const int lane = lane_id(), w = threadIdx.x / kWave;
  const int run = (B + kWavesMax - 1) / kWavesMax;  // tiles per wave
  const int r0 = min(B, w * run), r1 = min(B, r0 + run);
  const int ncb = (E + 1 + kWave - 1) / kWave;      // column blocks (E experts + received)
  for (int cb = blockIdx.x; cb < ncb; cb += gridDim.x) {
    const int c = cb * kWave + lane;
    const bool is_expert = c < E, is_recv = c == E;
    auto value = [&](int r) -> int {
      if (is_expert) return tile_counts[(int64_t)r * E + c];
      return is_recv ? tile_recv[r] : 0;
    };
    int sum = 0;
    for (int r = r0; r < r1; r += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = r + j < r1 ? value(r + j) : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) sum += v[j];
    }
    s_part[w][lane] = sum;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int ww = 0; ww < kWavesMax; ++ww) {
      const int x = s_part[ww][lane];
      before += ww < w ? x : 0;
      total += x;
    }
    __syncthreads();  // s_part is reused by the next column block
    int acc = before;
    for (int r = r0; r < r1; r += kScanBatch) {
      int v[kScanBatch];
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) v[j] = r + j < r1 ? value(r + j) : 0;
#pragma unroll
      for (int j = 0; j < kScanBatch; ++j) {
        if (r + j < r1) {
          if (is_expert) tile_base[(int64_t)(r + j) * E + c] = acc;
          else if (is_recv) recv_base[r + j] = acc;
        }
        acc += v[j];
      }
    }
    if (w == 0) {
      if (is_expert) expert_total[c] = total;
      else if (is_recv) *recv_total = total;
    }
  }
}

template <int K, int NW>
int tiles_for(int T) {
  return (T + Tile<K, NW>::tokens - 1) / Tile<K, NW>::tokens;
}

// Whether the many-tile path adds the tile-scan launch: without it, each
// thread of the second launch walks ceil(B / P) tiles, P = 1024 / E rounded
// up to a power of two, a chain of dependent load batches that grows with the
// tile count (78 us at 128K entries and 1024 experts).
inline bool use_tile_scan(int B, int E) {
  const int epad = E <= 1 ? 1 : 1 << (32 - __builtin_clz((unsigned)(E - 1)));
  const int P = epad >= kThreads ? 1 : kThreads / epad;
  return (B + P - 1) / P > kScanMinWalk;
}

// Most bytes the read-ahead covers: half of MI355X's 256 MiB last-level cache
// (dispatch's other traffic streams past it); larger token buffers never
// stay cached, and dispatch handles them with its grouped kernel.
constexpr int64_t kPrefetchMaxBytes = int64_t(128) << 20;
// Read-ahead workgroups per launch: one compute unit's memory path moves far
// less than HBM can (about 33-54 GB/s measured on MI355X), so the read-ahead
// is spread over most of the chip, at least 1024 lines (one load per lane of
// each of 16 waves) per workgroup.
constexpr int kPrefetchMaxBlocks = 224;
constexpr int64_t kPrefetchMinLinesPerBlock = int64_t(kWavesMax) * kWave;

// The read-ahead share [part, part + 1) of `parts` of a launch: nothing
// under a workgroup cap (the extra workgroups would exceed it).
inline Prefetch prefetch_part(const LayoutArgs &a, int cap, int part, int parts) {
  Prefetch pf{nullptr, 0, 0, 0};
  if (a.prefetch == nullptr || cap > 0) return pf;
  const int64_t lines = std::min<int64_t>(a.prefetch_bytes, kPrefetchMaxBytes) / 128;
  pf.p = (const uint32_t *)a.prefetch;
  pf.l0 = lines * part / parts;
  pf.l1 = lines * (part + 1) / parts;
  pf.blocks = (int)std::min<int64_t>((pf.l1 - pf.l0 + kPrefetchMinLinesPerBlock - 1) /
                                         kPrefetchMinLinesPerBlock, kPrefetchMaxBlocks);
  return pf;
}

template <int K, int NW, bool LOOP>
int layout_launch(const LayoutArgs &a, int B, unsigned G, int cap) {
  const size_t shm_rank = rank_lds_bytes(a.E, NW);
  if ((int64_t)a.T * K <= kFusedMaxEntries) {
    const Prefetch pf = LOOP ? Prefetch{nullptr, 0, 0, 0} : prefetch_part(a, cap, 0, 1);
    ep_layout_fused_tiles<K, NW, LOOP>
        <<<G + pf.blocks, kThreads, shm_rank + sizeof(int) * (size_t)(4 * a.E), a.stream>>>(
            a.topk_idx, a.T, a.E, a.A, B, a.counts, a.offsets, a.dst_slot, a.meta, a.num_recv,
            a.plan, pf);
    return launch_status();
  }
  // the read-ahead is split between the first and the last launch
  const Prefetch pf0 = LOOP ? Prefetch{nullptr, 0, 0, 0} : prefetch_part(a, cap, 0, 2);
  const Prefetch pf1 = LOOP ? Prefetch{nullptr, 0, 0, 0} : prefetch_part(a, cap, 1, 2);
  int32_t *tile_counts = (int32_t *)a.workspace;
  int32_t *tile_recv = tile_counts + (size_t)B * a.E;
  ep_layout_tile_histogram<K, NW, LOOP><<<G + pf0.blocks, kThreads, shm_rank, a.stream>>>(
      a.topk_idx, a.T, a.E, B, a.dst_slot, tile_counts, tile_recv, pf0);
  // each launch's status is read before the next launch can overwrite it
  if (int r = launch_status()) return r;
  const size_t shm_assign = sizeof(int) * (size_t)(3 * a.E);
  if (use_tile_scan(B, a.E)) {
    int32_t *tile_base = tile_recv + B;
    int32_t *expert_total = tile_base + (size_t)B * a.E;
    int32_t *recv_base = expert_total + a.E;
    int32_t *recv_total = recv_base + B;
    unsigned gs = (unsigned)((a.E + 1 + kWave - 1) / kWave);
    if (cap > 0 && gs > (unsigned)cap) gs = (unsigned)cap;
    ep_layout_tile_scan<<<gs, kThreads, 0, a.stream>>>(tile_counts, tile_recv, B, a.E, tile_base,
                                                        expert_total, recv_base, recv_total);
    if (int r = launch_status()) return r;
    const TileScan scan{tile_base, expert_total, recv_base, recv_total};
    ep_layout_tile_assign<K, NW, LOOP, true><<<G + pf1.blocks, kThreads, shm_assign, a.stream>>>(
        a.T, a.E, a.A, B, tile_counts, tile_recv, scan, a.counts, a.offsets, a.dst_slot, a.meta,
        a.num_recv, a.plan, pf1);
  } else {
    ep_layout_tile_assign<K, NW, LOOP, false>
        <<<G + pf1.blocks, kThreads, shm_assign, a.stream>>>(
            a.T, a.E, a.A, B, tile_counts, tile_recv, TileScan{}, a.counts, a.offsets,
            a.dst_slot, a.meta, a.num_recv, a.plan, pf1);
  }
  return launch_status();
}

template <int K, int NW>
int layout_impl(const LayoutArgs &a) {
  const int B = tiles_for<K, NW>(a.T);
  const int cap = stream_workgroup_limit(a.stream);
  if (B <= 1) {
    const size_t shm_rank = rank_lds_bytes(a.E, NW);
    const Prefetch pf = prefetch_part(a, cap, 0, 1);
    ep_layout_single_tile<K, NW>
        <<<1 + pf.blocks, kThreads, shm_rank + sizeof(int) * (size_t)(2 * a.E), a.stream>>>(
            a.topk_idx, a.T, a.E, a.A, a.counts, a.offsets, a.dst_slot, a.meta, a.num_recv,
            a.plan, pf);
    return launch_status();
  }
  if (cap > 0 && cap < B) return layout_launch<K, NW, true>(a, B, (unsigned)cap, cap);
  return layout_launch<K, NW, false>(a, B, (unsigned)B, cap);
}

template <int K>
int layout_k(const LayoutArgs &a) {
  switch (tile_waves(a.E)) {
    case 16: return layout_impl<K, 16>(a);
    case 8: return layout_impl<K, 8>(a);
    default: return layout_impl<K, 4>(a);
  }
}

// Most workgroups of the fused layout + dispatch launch, one per compute
// unit: each repeats the ranking, so more only add LDS work. Measured on
// MI355X (decode step, 128 tokens, top-8, hidden 7168, with combine): 13.5 /
// 12.1 / 12.8 / 17.5 us per step at 128 / 256 / 512 / 1024 workgroups, against
// 15.8 with layout and dispatch launched separately.
constexpr int kFusedDispatchMaxBlocks = 256;

template <int K, int NW>
int layout_dispatch_impl(const LayoutArgs &l, const DispatchArgs &d, int row_chunks,
                         int scale_chunks) {
  if (tiles_for<K, NW>(l.T) > 1) return -3;  // more than one tile: not fused
  const int cap = stream_workgroup_limit(l.stream);
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int64_t units = (int64_t)l.T * K * slices;
  int64_t blocks = (units + kWavesMax - 1) / kWavesMax;
  if (blocks > kFusedDispatchMaxBlocks) blocks = kFusedDispatchMaxBlocks;
  if (cap > 0 && blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const size_t shm = rank_lds_bytes(l.E, NW) + sizeof(int) * ((size_t)l.E + kThreads);
  const bool fwd_w = d.topk_weights != nullptr && d.expand_weights != nullptr;
  auto go = [&](auto wide, auto counted, int64_t grid) {
    ep_layout_dispatch_tile<K, NW, decltype(wide)::value, decltype(counted)::value>
        <<<(unsigned)grid, kThreads, shm, l.stream>>>(
            l.topk_idx, l.T, l.E, l.A, l.counts, l.offsets, l.dst_slot, l.meta, l.num_recv,
            (const u32x4 *)d.x, row_chunks, (const u32x4 *)d.x_scales, scale_chunks,
            d.topk_weights, d.capacity, (u32x4 *)d.expand_x, (u32x4 *)d.expand_scales,
            fwd_w ? d.expand_weights : nullptr, fast_div((uint32_t)slices));
  };
  if (cap > 0) go(std::false_type{}, std::false_type{}, blocks);
  else if (l.A == 1)  // workgroup 0 lays out, the others copy
    go(std::true_type{}, std::true_type{}, (units > 0 ? std::min<int64_t>(blocks, kFusedDispatchMaxBlocks - 1) : 0) + 1);
  else go(std::true_type{}, std::false_type{}, blocks);
  return launch_status();
}

template <int K, int NW>
int layout_dispatch_compact_impl(const LayoutArgs &l, const CompactDispatchArgs &d) {
  if (tiles_for<K, NW>(l.T) > 1) return -3;  // more than one tile: not fused
  const int cap = stream_workgroup_limit(l.stream);
  const int row_chunks = (int)(d.row_bytes / 16);
  const int64_t slices = (row_chunks + kWave - 1) / kWave;
  const int64_t units = (int64_t)l.T * slices;
  int64_t blocks = (units + kWavesMax - 1) / kWavesMax;
  if (blocks > kFusedDispatchMaxBlocks) blocks = kFusedDispatchMaxBlocks;
  if (cap > 0 && blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const size_t shm = rank_lds_bytes(l.E, NW) + sizeof(int) * (size_t)l.E;
  auto go = [&](auto wide) {
    ep_layout_dispatch_compact_tile<K, NW, decltype(wide)::value>
        <<<(unsigned)blocks, kThreads, shm, l.stream>>>(
            l.topk_idx, l.T, l.E, l.A, l.counts, l.offsets, l.dst_slot, l.meta, l.num_recv,
            (const u32x4 *)d.x, row_chunks, d.x_scales, (int)d.scale_cols, d.topk_weights,
            (u32x4 *)d.recv_x, d.recv_scales, d.recv_topk_idx, d.recv_topk_weights,
            fast_div((uint32_t)slices));
  };
  if (cap > 0) go(std::false_type{});
  else go(std::true_type{});
  return launch_status();
}

template <int K>
int layout_dispatch_compact_k(const LayoutArgs &l, const CompactDispatchArgs &d) {
  switch (tile_waves(l.E)) {
    case 16: return layout_dispatch_compact_impl<K, 16>(l, d);
    case 8: return layout_dispatch_compact_impl<K, 8>(l, d);
    default: return layout_dispatch_compact_impl<K, 4>(l, d);
  }
}

template <int K>
int layout_dispatch_k(const LayoutArgs &l, const DispatchArgs &d, int row_chunks,
                      int scale_chunks) {
  switch (tile_waves(l.E)) {
    case 16: return layout_dispatch_impl<K, 16>(l, d, row_chunks, scale_chunks);
    case 8: return layout_dispatch_impl<K, 8>(l, d, row_chunks, scale_chunks);
    default: return layout_dispatch_impl<K, 4>(l, d, row_chunks, scale_chunks);
  }
}

template <int K>
size_t workspace_k(int T, int E) {
  int B;
  switch (tile_waves(E)) {
    case 16: B = tiles_for<K, 16>(T); break;
    case 8: B = tiles_for<K, 8>(T); break;
    default: B = tiles_for<K, 4>(T); break;
  }
  if (B <= 1 || (int64_t)T * K <= kFusedMaxEntries) return 0;
  // tile counts [B][E] and received tokens [B]; with the tile scan also its
  // prefixes [B][E], expert totals [E], received prefixes [B] and total
  const size_t ints = use_tile_scan(B, E) ? 2 * (size_t)B * E + 2 * (size_t)B + E + 1
                                          : (size_t)B * E + B;
  return (ints * sizeof(int32_t) + 255) & ~(size_t)255;
}

}  // namespace

#define EP_LAYOUT_CASE(K) \
  case K:                 \
    return layout_k<K>(a);

int launch_layout(const LayoutArgs &a) {
  switch (a.K) { EP_FOR_EACH_TOPK(EP_LAYOUT_CASE) default: return -2; }
}

#define EP_LAYOUT_DISPATCH_CASE(K) \
  case K:                          \
    return layout_dispatch_k<K>(l, d, row_chunks, scale_chunks);

int launch_layout_dispatch(const LayoutArgs &l, const DispatchArgs &d, int row_chunks,
                           int scale_chunks) {
  switch (l.K) { EP_FOR_EACH_TOPK(EP_LAYOUT_DISPATCH_CASE) default: return -2; }
}

#define EP_LAYOUT_DISPATCH_COMPACT_CASE(K) \
  case K:                                  \
    return layout_dispatch_compact_k<K>(l, d);

int launch_layout_dispatch_compact(const LayoutArgs &l, const CompactDispatchArgs &d) {
  switch (l.K) { EP_FOR_EACH_TOPK(EP_LAYOUT_DISPATCH_COMPACT_CASE) default: return -2; }
}

#define EP_WS_CASE(K) \
  case K:             \
    return workspace_k<K>(T, E);

size_t layout_workspace(int T, int K, int E) {
  switch (K) { EP_FOR_EACH_TOPK(EP_WS_CASE) default: return 0; }
}

}  // namespace ep

// Fixed device scratch for ep_layout_noalloc: the workspace of the many-tile
// launches (per-tile histograms, received-token counts and tile-scan
// prefixes) for callers that cannot allocate one. Every GPU holds its own
// copy for the life of the process; every call on one GPU shares it, so two
// such calls in flight on one GPU at once race. Nothing in it needs to start
// at zero: each launch writes every word it later reads.
static __device__ __align__(256) unsigned char scratch[EP_LAYOUT_SCRATCH_BYTES];

namespace ep {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (guarded)
}  // namespace

// Device address of the current device's `scratch`, looked up on the first
// call on each device, with that device current. The host-side name of the
// array is only a registration handle: kernels must be given this address.
hipError_t layout_scratch(int device, void **ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace ep
