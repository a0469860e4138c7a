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
// Design (MI355X): entries are cut into tiles of whole tokens, at most 1024
// entries, one workgroup of 16 wave64s per tile, one entry per thread.
//   1. Inside a wavefront, lanes holding the same expert are grouped with a
//      ballot loop (one iteration per distinct expert of the wave); a lane's
//      rank is the popcount of its group's ballot below it (mbcnt).
//   2. Per-wave group sizes go to an LDS histogram [16 waves][E]; a scan over
//      the 16 waves gives each wave its base, so rank-in-tile is exact.
//   3. A tile's per-expert totals are written to the workspace. A second
//      launch reduces, per expert, the totals of earlier tiles (prefix) and
//      of all tiles (count), pads each count to the alignment, scans over
//      experts in LDS, and writes slot = offset + prefix + rank-in-tile.
// A single tile (small T*K) runs both halves in one launch with no
// workspace. Integer LDS atomics are never used, so results do not depend
// on scheduling.
#include "ep_device.hpp"
#include "ep_launch.hpp"

namespace ep {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kRankBits = 10;  // rank inside a tile < 1024

template <int K>
struct Tile {
  static constexpr int tokens = kThreads / K;  // whole tokens per tile
  static constexpr int entries = tokens * K;   // <= kThreads
};

struct EntryRank {
  int e;     // expert of this thread's entry, -1 if masked or absent
  int rank;  // entries of the same expert earlier in the tile
};

// Steps 1 and 2 above. s_wcnt: uint16 [kWaves][E]; s_total: int [E] receives
// the tile's per-expert counts.
template <int K>
__device__ EntryRank tile_rank(const int32_t *__restrict__ topk_idx, int64_t t0, int ntok, int E,
                               uint16_t *s_wcnt, int *s_total) {
  const int tid = threadIdx.x, lane = lane_id(), w = tid / kWave;
  for (int i = tid; i < kWaves * E; i += kThreads) s_wcnt[i] = 0;
  int e = -1;
  if (tid < ntok * K) {
    const int v = topk_idx[t0 * K + tid];
    e = (v >= 0 && v < E) ? v : -1;
  }
  __syncthreads();
  int rank = 0;
  uint64_t pending = ballot(e >= 0);
  while (pending) {  // wave-uniform: one pass per distinct expert in the wave
    const int leader = __builtin_ctzll(pending);
    const int le = read_lane(e, leader);
    const uint64_t group = ballot(e == le);
    if (e == le) rank = count_below(group);
    if (lane == leader) s_wcnt[w * E + le] = (uint16_t)__popcll(group);
    pending &= ~group;
  }
  __syncthreads();
  for (int ex = tid; ex < E; ex += kThreads) {
    int run = 0;
    for (int ww = 0; ww < kWaves; ++ww) {
      const int c = s_wcnt[ww * E + ex];
      s_wcnt[ww * E + ex] = (uint16_t)run;
      run += c;
    }
    s_total[ex] = run;
  }
  __syncthreads();
  if (e >= 0) rank += s_wcnt[w * E + e];
  return {e, rank};
}

// Thread j (< ntok) gets 1 if token j of the tile has an unmasked entry.
// s_tok: int [Tile<K>::tokens].
template <int K>
__device__ int tile_token_flag(int e, int ntok, int *s_tok) {
  const int tid = threadIdx.x;
  if (tid < Tile<K>::tokens) s_tok[tid] = 0;
  __syncthreads();
  if (e >= 0) s_tok[tid / K] = 1;  // every writer stores the same value
  __syncthreads();
  const int f = (tid < ntok) ? s_tok[tid] : 0;
  __syncthreads();
  return f;
}

// Final slots of the tile's entries and their metadata rows. `slot` is the
// entry's slot or -1; `flag` is thread j's token flag; `vpre` the number of
// received tokens before this tile.
template <int K>
__device__ void write_slots_and_meta(int64_t t0, int ntok, int slot, int flag, int vpre,
                                     int32_t *__restrict__ dst_slot,
                                     int32_t *__restrict__ meta, int *s_tok, int *s_tmp) {
  const int tid = threadIdx.x;
  int n_flagged;
  const int tok_rank = block_exclusive_scan<kThreads>(flag, s_tmp, n_flagged);
  if (tid < ntok) s_tok[tid] = flag ? vpre + tok_rank : -1;
  __syncthreads();
  if (tid < ntok * K) {
    dst_slot[t0 * K + tid] = slot;
    const int j = tid / K, k = tid - j * K;
    const int row = s_tok[j];
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

__host__ __device__ constexpr size_t wcnt_bytes(int E) {
  return ((size_t)kWaves * E * sizeof(uint16_t) + 15) & ~(size_t)15;
}

// One launch for T*K that fits a single tile (including T = 0).
template <int K>
__global__ __launch_bounds__(kThreads) void ep_layout_single_tile(
    const int32_t *__restrict__ topk_idx, int T, int E, int A, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *s_wcnt = (uint16_t *)smem;
  int *s_total = (int *)(smem + wcnt_bytes(E));
  int *s_off = s_total + E;  // E + 1
  __shared__ int s_tok[Tile<K>::tokens];
  __shared__ int s_tmp[kWaves];
  const int tid = threadIdx.x;
  const int ntok = T;

  const EntryRank r = tile_rank<K>(topk_idx, 0, ntok, E, s_wcnt, s_total);
  const int cnt = tid < E ? s_total[tid] : 0;
  const int padded = ((cnt + A - 1) / A) * A;
  int rows;
  const int off = block_exclusive_scan<kThreads>(padded, s_tmp, rows);
  if (tid < E) {
    s_off[tid] = off;
    counts[tid] = cnt;
    offsets[tid] = off;
  }
  if (tid == 0) offsets[E] = rows;
  __syncthreads();
  const int slot = r.e >= 0 ? s_off[r.e] + r.rank : -1;
  const int flag = tile_token_flag<K>(r.e, ntok, s_tok);
  int nrecv;
  block_exclusive_scan<kThreads>(flag, s_tmp, nrecv);
  if (tid == 0) *num_recv = nrecv;
  write_slots_and_meta<K>(0, ntok, slot, flag, 0, dst_slot, meta, s_tok, s_tmp);
}

// First launch of the multi-tile path: per-tile histograms and ranks.
// dst_slot temporarily holds (expert << kRankBits | rank-in-tile), or -1.
template <int K>
__global__ __launch_bounds__(kThreads) void ep_layout_tile_histogram(
    const int32_t *__restrict__ topk_idx, int T, int E, int32_t *__restrict__ dst_slot,
    int32_t *__restrict__ tile_counts, int32_t *__restrict__ tile_recv) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t *s_wcnt = (uint16_t *)smem;
  int *s_total = (int *)(smem + wcnt_bytes(E));
  __shared__ int s_tok[Tile<K>::tokens];
  __shared__ int s_tmp[kWaves];
  const int tid = threadIdx.x, b = blockIdx.x;
  const int64_t t0 = (int64_t)b * Tile<K>::tokens;
  const int ntok = (int)min((int64_t)Tile<K>::tokens, (int64_t)T - t0);

  const EntryRank r = tile_rank<K>(topk_idx, t0, ntok, E, s_wcnt, s_total);
  if (tid < ntok * K) dst_slot[t0 * K + tid] = r.e >= 0 ? (r.e << kRankBits) | r.rank : -1;
  for (int ex = tid; ex < E; ex += kThreads) tile_counts[(int64_t)b * E + ex] = s_total[ex];
  const int flag = tile_token_flag<K>(r.e, ntok, s_tok);
  int nflag;
  block_exclusive_scan<kThreads>(flag, s_tmp, nflag);
  if (tid == 0) tile_recv[b] = nflag;
}

// Second launch: offsets, final slots and metadata for tile blockIdx.x.
template <int K>
__global__ __launch_bounds__(kThreads) void ep_layout_tile_assign(
    int T, int E, int A, int num_tiles, const int32_t *__restrict__ tile_counts,
    const int32_t *__restrict__ tile_recv, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ dst_slot, int32_t *__restrict__ meta,
    int32_t *__restrict__ num_recv) {
  __shared__ int s_pre[kThreads];
  __shared__ int s_tot[kThreads];
  __shared__ int s_tok[Tile<K>::tokens];
  __shared__ int s_tmp[kWaves];
  extern __shared__ __align__(16) unsigned char smem[];
  int *s_base = (int *)smem;  // E
  int *s_off = s_base + E;    // E
  const int tid = threadIdx.x, b = blockIdx.x;

  // Per expert: entries in tiles before b, and in all tiles. P threads share
  // an expert so that all the loads of a thread are in flight together.
  const int epad = E <= 1 ? 1 : 1 << (32 - __builtin_clz((unsigned)(E - 1)));
  const int P = kThreads / epad;
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
  s_pre[tid] = pre;
  s_tot[tid] = tot;
  __syncthreads();
  int base = 0, cnt = 0;
  if (tid < E) {
    for (int j = 0; j < P; ++j) {
      base += s_pre[j * epad + tid];
      cnt += s_tot[j * epad + tid];
    }
  }
  const int padded = ((cnt + A - 1) / A) * A;
  int rows;
  const int off = block_exclusive_scan<kThreads>(padded, s_tmp, rows);
  if (tid < E) {
    s_base[tid] = base;
    s_off[tid] = off;
  }
  if (b == 0) {
    if (tid < E) {
      counts[tid] = cnt;
      offsets[tid] = off;
    }
    if (tid == 0) offsets[E] = rows;
  }

  // Received tokens before this tile, and in all tiles.
  int vpre = 0, vtot = 0;
  for (int bb = tid; bb < num_tiles; bb += kThreads) {
    const int c = tile_recv[bb];
    vtot += c;
    vpre += bb < b ? c : 0;
  }
  int vpre_all, vtot_all;
  block_exclusive_scan<kThreads>(vpre, s_tmp, vpre_all);
  block_exclusive_scan<kThreads>(vtot, s_tmp, vtot_all);
  if (b == 0 && tid == 0) *num_recv = vtot_all;

  const int64_t t0 = (int64_t)b * Tile<K>::tokens;
  const int ntok = (int)min((int64_t)Tile<K>::tokens, (int64_t)T - t0);
  int slot = -1, e = -1;
  if (tid < ntok * K) {
    const int p = dst_slot[t0 * K + tid];
    if (p >= 0) {
      e = p >> kRankBits;
      slot = s_off[e] + s_base[e] + (p & ((1 << kRankBits) - 1));
    }
  }
  const int flag = tile_token_flag<K>(e, ntok, s_tok);
  write_slots_and_meta<K>(t0, ntok, slot, flag, vpre_all, dst_slot, meta, s_tok, s_tmp);
}

template <int K>
int tiles_for(int T) {
  return (T + Tile<K>::tokens - 1) / Tile<K>::tokens;
}

template <int K>
int layout_impl(const LayoutArgs &a) {
  const int B = tiles_for<K>(a.T);
  const size_t shm_hist = wcnt_bytes(a.E) + sizeof(int) * (size_t)(2 * a.E + 1);
  if (B <= 1) {
    ep_layout_single_tile<K><<<1, kThreads, shm_hist, a.stream>>>(
        a.topk_idx, a.T, a.E, a.A, a.counts, a.offsets, a.dst_slot, a.meta, a.num_recv);
  } else {
    int32_t *tile_counts = (int32_t *)a.workspace;
    int32_t *tile_recv = tile_counts + (size_t)B * a.E;
    ep_layout_tile_histogram<K><<<B, kThreads, shm_hist, a.stream>>>(
        a.topk_idx, a.T, a.E, a.dst_slot, tile_counts, tile_recv);
    ep_layout_tile_assign<K><<<B, kThreads, sizeof(int) * (size_t)(2 * a.E), a.stream>>>(
        a.T, a.E, a.A, B, tile_counts, tile_recv, a.counts, a.offsets, a.dst_slot, a.meta,
        a.num_recv);
  }
  return launch_status();
}

template <int K>
size_t workspace_impl(int T, int E) {
  const int B = tiles_for<K>(T);
  return B <= 1 ? 0 : (((size_t)B * E + B) * sizeof(int32_t) + 255) & ~(size_t)255;
}

}  // namespace

#define EP_LAYOUT_CASE(K) \
  case K:                 \
    return layout_impl<K>(a);

int launch_layout(const LayoutArgs &a) {
  switch (a.K) { EP_FOR_EACH_TOPK(EP_LAYOUT_CASE) default: return -2; }
}

#define EP_WS_CASE(K) \
  case K:             \
    return workspace_impl<K>(T, E);

size_t layout_workspace(int T, int K, int E) {
  switch (K) { EP_FOR_EACH_TOPK(EP_WS_CASE) default: return 0; }
}

}  // namespace ep
