/*
 * CPU oracle for MoE expert-parallel layout, dispatch and combine, taken at
 * one GPU's share (every expert local, a world of one).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct
 * reference that the GPU path is checked against. Only the test-suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path never calls it. It is plain C99, built with gcc and
 * -ffp-contract=off, includes no HIP header and shares no code with the GPU
 * library.
 *
 * Sources (the pages this follows):
 *   [DeepEP]  "DeepEP 整体架构分析" (DeepEP overall architecture): the EPHandle
 *             structure (do_expand, expert_alignment, psum_num_recv_tokens_per_expert,
 *             num_unaligned_recv_tokens_perpert, recv_src_metadata,
 *             dst_buffer_slot_idx, num_recv_tokens, num_expanded_tokens) and
 *             the dispatch / combine data-flow figure (notify warps count per
 *             expert and compute target slots; the copy epilogue writes rows;
 *             the reduce epilogue weights rows by topk_weights).
 *   [MORI]    "MORI JIT v2", section 3.7 (dtype is a transport attribute):
 *             dispatch only moves the payload bytes, fp8 / fp4 rows travel
 *             as one-byte elements that arrive already quantised, combine
 *             reduces and rejects byte dtypes.
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes of the repository):
 *   - order inside an expert segment: stable, token-major (t, then k);
 *   - the per-expert prefix sum is exclusive with E+1 entries, each segment
 *     padded up to a multiple of expert_alignment; an empty expert gets no
 *     rows; the last entry is num_expanded_tokens;
 *   - an entry whose expert id lies outside [0, E) is masked: it is not
 *     counted, its slot is -1, combine skips it;
 *   - recv_src_metadata row i = [source token, source rank (0 in a world of
 *     one), slot of k = 0 .. K-1] for the i-th token (ascending) that has
 *     at least one unmasked entry; rows past num_recv are not written;
 *   - combine accumulates in fp32, starting at +0.0, in k order, each
 *     product and each sum rounded separately, adds the bias (if any) last,
 *     then rounds to bf16 with round-to-nearest-even (NaN becomes a quiet
 *     NaN with its sign); a null weight pointer means weight 1.
 *
 * Parity is pinned (tests in tests/test_oracle_*.py) by brute force on tiny
 * inputs, by library routines (bincount, stable argsort, fancy indexing), by
 * invariants (counts sum, per-expert permutation, alignment, capacity bound),
 * by a float64 reference with a rigorous fp32 error bound, by bit-exact
 * special cases (K = 1, identity-expert round trip) and by hand-worked
 * examples under tests/golden/.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#if defined(__HIP__) || defined(__HIPCC__) || defined(__CUDACC__)
#error "the oracle must be compiled by a plain host C compiler"
#endif

/* ---------------------------------------------------------------------- */
/* Layout: counts, aligned exclusive prefix, destination slots, metadata.  */
/* ---------------------------------------------------------------------- */

/*
 * Step 1, per-expert token count ([DeepEP] EPHandle
 * num_unaligned_recv_tokens_perpert; the notify warps of the dispatch
 * data-flow figure count entries per expert).
 */
static void count_per_expert(const int32_t *topk_idx, int64_t n_entries,
                             int32_t E, int32_t *counts) {
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < n_entries; ++i) {
    int32_t e = topk_idx[i];
    if (e >= 0 && e < E) counts[e] += 1;
  }
}

/*
 * Step 2, exclusive prefix sum of the counts with each expert's segment
 * rounded up to a multiple of expert_alignment ([DeepEP] EPHandle
 * psum_num_recv_tokens_per_expert, expert_alignment, num_expanded_tokens).
 */
static void aligned_exclusive_prefix(const int32_t *counts, int32_t E,
                                     int32_t A, int32_t *offsets) {
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) {
    int32_t padded = ((counts[e] + A - 1) / A) * A;
    offsets[e + 1] = offsets[e] + padded;
  }
}

/*
 * Step 3, destination slot of every (token, k) ([DeepEP] EPHandle
 * dst_buffer_slot_idx; the notify warps compute each target slot): walk the
 * entries in token-major order and hand out the next free row of the
 * expert's segment.
 */
static void assign_slots(const int32_t *topk_idx, int32_t T, int32_t K,
                         int32_t E, const int32_t *offsets, int32_t *dst_slot) {
  int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t k = 0; k < K; ++k) {
      int64_t i = (int64_t)t * K + k;
      int32_t e = topk_idx[i];
      if (e >= 0 && e < E) {
        dst_slot[i] = cursor[e];
        cursor[e] += 1;
      } else {
        dst_slot[i] = -1;
      }
    }
  }
  free(cursor);
}

/*
 * Step 4, receive-side source metadata ([DeepEP] EPHandle recv_src_metadata
 * [num_recv_tokens, topk + 2], "source token index + slot"; num_recv_tokens).
 */
static int32_t build_recv_metadata(const int32_t *dst_slot, int32_t T, int32_t K,
                                   int32_t *meta) {
  int32_t i = 0;
  for (int32_t t = 0; t < T; ++t) {
    int any = 0;
    for (int32_t k = 0; k < K; ++k)
      if (dst_slot[(int64_t)t * K + k] >= 0) any = 1;
    if (!any) continue;
    int32_t *row = meta + (int64_t)i * (K + 2);
    row[0] = t;
    row[1] = 0; /* source rank: a world of one */
    for (int32_t k = 0; k < K; ++k) row[2 + k] = dst_slot[(int64_t)t * K + k];
    i += 1;
  }
  return i;
}

/*
 * The whole layout pass. Returns 0, or -1 when an argument is out of range.
 * counts[E], offsets[E+1], dst_slot[T*K], meta[T*(K+2)] (only the first
 * *num_recv rows are written), num_recv[1].
 */
int oracle_layout(const int32_t *topk_idx, int32_t T, int32_t K, int32_t E,
                  int32_t A, int32_t *counts, int32_t *offsets,
                  int32_t *dst_slot, int32_t *meta, int32_t *num_recv) {
  if (T < 0 || K < 1 || E < 1 || A < 1) return -1;
  count_per_expert(topk_idx, (int64_t)T * K, E, counts);
  aligned_exclusive_prefix(counts, E, A, offsets);
  assign_slots(topk_idx, T, K, E, offsets, dst_slot);
  *num_recv = build_recv_metadata(dst_slot, T, K, meta);
  return 0;
}

/* bf16 is the upper half of an IEEE binary32. */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* binary32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN. */
static uint16_t float_to_bf16_bits_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
    return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------------------------- */
/* Dispatch: move bytes into the expert-major expand buffer.               */
/* ---------------------------------------------------------------------- */

/*
 * [MORI] 3.7 and [DeepEP] dispatch copy epilogue ("token data + sf"):
 * expand_x[dst, :] = x[t, :] as raw bytes for every unmasked (t, k);
 * for fp8 the scale row travels with it, and the router weight travels
 * with the row when both weight pointers are given. Rows that no entry
 * points at (alignment padding) are not touched.
 */
int oracle_dispatch(const uint8_t *x, int64_t row_bytes, const uint8_t *x_scales,
                    int64_t scale_row_bytes, const float *topk_weights,
                    const int32_t *dst_slot, int32_t T, int32_t K,
                    int64_t capacity_rows, uint8_t *expand_x,
                    uint8_t *expand_scales, float *expand_weights) {
  if (T < 0 || K < 1 || row_bytes < 0) return -1;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t k = 0; k < K; ++k) {
      int64_t d = dst_slot[(int64_t)t * K + k];
      if (d < 0) continue;
      if (d >= capacity_rows) return -1;
      memcpy(expand_x + d * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);
      if (x_scales && expand_scales)
        memcpy(expand_scales + d * scale_row_bytes,
               x_scales + (int64_t)t * scale_row_bytes, (size_t)scale_row_bytes);
      if (topk_weights && expand_weights)
        expand_weights[d] = topk_weights[(int64_t)t * K + k];
    }
  }
  return 0;
}

/*
 * Non-expand dispatch ([DeepEP] EPHandle do_expand = false; the dispatch
 * copy epilogue writes recv_x, recv_topk_idx and recv_topk_weights): one row
 * per received token, in receive order. For i < num_recv, with
 * t = recv_src_metadata[i][0]:
 *   recv_x[i] = x[t] (bytes), recv_scales[i] = x_scales[t] (if given),
 *   recv_topk_idx[i][k] = topk_idx[t][k] where dst_slot[t][k] >= 0, else -1,
 *   recv_topk_weights[i][k] = topk_weights[t][k] (if given).
 */
int oracle_dispatch_compact(const uint8_t *x, int64_t row_bytes, const uint8_t *x_scales,
                            int64_t scale_row_bytes, const int32_t *topk_idx,
                            const float *topk_weights, const int32_t *dst_slot,
                            const int32_t *meta, int32_t num_recv, int32_t T, int32_t K,
                            uint8_t *recv_x, uint8_t *recv_scales, int32_t *recv_topk_idx,
                            float *recv_topk_weights) {
  if (num_recv < 0 || num_recv > T || K < 1 || row_bytes < 0) return -1;
  for (int32_t i = 0; i < num_recv; ++i) {
    int32_t t = meta[(int64_t)i * (K + 2)];
    if (t < 0 || t >= T) return -1;
    memcpy(recv_x + (int64_t)i * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);
    if (x_scales && recv_scales)
      memcpy(recv_scales + (int64_t)i * scale_row_bytes, x_scales + (int64_t)t * scale_row_bytes,
             (size_t)scale_row_bytes);
    for (int32_t k = 0; k < K; ++k) {
      int64_t tk = (int64_t)t * K + k;
      recv_topk_idx[(int64_t)i * K + k] = dst_slot[tk] >= 0 ? topk_idx[tk] : -1;
      if (topk_weights && recv_topk_weights)
        recv_topk_weights[(int64_t)i * K + k] = topk_weights[tk];
    }
  }
  return 0;
}

/*
 * Non-expand combine in a world of one: the expert side returns one row per
 * received token with that token's experts already reduced, so the combine
 * only puts rows back in token order and adds the bias: out[t] =
 * bf16(float(y[i]) + float(bias[t])) for the token t of receive row i, and
 * out[t] = bf16(+0.0 + float(bias[t])) for a token with no unmasked entry;
 * without a bias, out[t] = y[i] (the same bits) or +0.
 */
int oracle_combine_compact(const uint16_t *y, int32_t H, const uint16_t *bias,
                           const int32_t *dst_slot, const int32_t *meta, int32_t num_recv,
                           int32_t T, int32_t K, uint16_t *out) {
  if (num_recv < 0 || num_recv > T || K < 1 || H < 0) return -1;
  int32_t *row_of = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  for (int32_t t = 0; t < T; ++t) row_of[t] = -1;
  for (int32_t i = 0; i < num_recv; ++i) {
    int32_t t = meta[(int64_t)i * (K + 2)];
    if (t < 0 || t >= T) {
      free(row_of);
      return -1;
    }
    row_of[t] = i;
  }
  for (int32_t t = 0; t < T; ++t) {
    int any = 0;
    for (int32_t k = 0; k < K; ++k)
      if (dst_slot[(int64_t)t * K + k] >= 0) any = 1;
    int32_t i = any ? row_of[t] : -1;
    for (int32_t h = 0; h < H; ++h) {
      uint16_t v;
      if (bias) {
        float acc = i >= 0 ? bf16_bits_to_float(y[(int64_t)i * H + h]) : 0.0f;
        acc = acc + bf16_bits_to_float(bias[(int64_t)t * H + h]);
        v = float_to_bf16_bits_rne(acc);
      } else {
        v = i >= 0 ? y[(int64_t)i * H + h] : (uint16_t)0;
      }
      out[(int64_t)t * H + h] = v;
    }
  }
  free(row_of);
  return 0;
}

/*
 * The same non-expand combine for binary32 rows ("MORI JIT v2", section 3.7:
 * combine takes bf16 or fp32 rows and writes the same type): for the token t
 * of receive row i, out[t] = y[i] + bias[t] in binary32 (one rounded add per
 * value); a token with no unmasked entry gets +0.0 + bias[t]; without a bias,
 * out[t] = y[i] value for value, or +0.0. y is fp32 [>= num_recv, H], bias
 * fp32 [T, H] or NULL, out fp32 [T, H].
 */
int oracle_combine_compact_f32(const float *y, int32_t H, const float *bias,
                               const int32_t *dst_slot, const int32_t *meta, int32_t num_recv,
                               int32_t T, int32_t K, float *out) {
  if (num_recv < 0 || num_recv > T || K < 1 || H < 0) return -1;
  /* receive row of each token, from the metadata's token column */
  int32_t *recv_row = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  for (int32_t t = 0; t < T; ++t) recv_row[t] = -1;
  for (int32_t i = 0; i < num_recv; ++i) {
    int32_t t = meta[(int64_t)i * (K + 2)];
    if (t < 0 || t >= T) {
      free(recv_row);
      return -1;
    }
    recv_row[t] = i;
  }
  for (int32_t t = 0; t < T; ++t) {
    int received = 0;
    for (int32_t k = 0; k < K; ++k)
      if (dst_slot[(int64_t)t * K + k] >= 0) received = 1;
    const float *row = received && recv_row[t] >= 0 ? y + (int64_t)recv_row[t] * H : NULL;
    for (int32_t h = 0; h < H; ++h) {
      float v = row ? row[h] : 0.0f;
      if (bias) v = v + bias[(int64_t)t * H + h];
      out[(int64_t)t * H + h] = v;
    }
  }
  free(recv_row);
  return 0;
}

/*
 * Optional clean-up of the expand layout: the alignment padding rows of each
 * expert segment, [offsets[e] + counts[e], offsets[e+1]), are set to zero in
 * expand_x (and in expand_scales / expand_weights when given), so a consumer
 * that walks whole aligned segments reads zeros there. Real rows are not
 * touched.
 */
int oracle_zero_padding(uint8_t *expand_x, int64_t row_bytes, uint8_t *expand_scales,
                        int64_t scale_row_bytes, float *expand_weights,
                        const int32_t *counts, const int32_t *offsets, int32_t E,
                        int64_t capacity_rows) {
  if (E < 1 || row_bytes < 0) return -1;
  for (int32_t e = 0; e < E; ++e) {
    for (int64_t r = (int64_t)offsets[e] + counts[e]; r < offsets[e + 1]; ++r) {
      if (r >= capacity_rows) return -1;
      memset(expand_x + r * row_bytes, 0, (size_t)row_bytes);
      if (expand_scales) memset(expand_scales + r * scale_row_bytes, 0, (size_t)scale_row_bytes);
      if (expand_weights) expand_weights[r] = 0.0f;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Combine: weighted gather-reduce back to token order.                    */
/* ---------------------------------------------------------------------- */

/*
 * [DeepEP] combine reduce epilogue (reduce weighted by topk_weights, plus a
 * bias) and [MORI] 3.7 (combine reduces bf16 rows): for each token t and
 * channel h,
 *   acc = +0.0f; for k = 0 .. K-1 with dst >= 0: acc = acc + w[t,k] * y[dst,h]
 *   if bias: acc = acc + bias[t,h]
 * in binary32, then out[t,h] = bf16_rne(acc). bias is bf16 [T, H] or NULL.
 */
int oracle_combine(const uint16_t *y, int32_t H, const float *topk_weights,
                   const uint16_t *bias, const int32_t *dst_slot, int32_t T, int32_t K,
                   int64_t capacity_rows, uint16_t *out) {
  if (T < 0 || K < 1 || H < 0) return -1;
  for (int32_t t = 0; t < T; ++t) {
    const int32_t *d = dst_slot + (int64_t)t * K;
    for (int32_t k = 0; k < K; ++k)
      if (d[k] >= capacity_rows) return -1;
    for (int32_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (int32_t k = 0; k < K; ++k) {
        if (d[k] < 0) continue;
        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;
        float v = bf16_bits_to_float(y[(int64_t)d[k] * H + h]);
        float prod = w * v;
        acc = acc + prod;
      }
      if (bias) acc = acc + bf16_bits_to_float(bias[(int64_t)t * H + h]);
      out[(int64_t)t * H + h] = float_to_bf16_bits_rne(acc);
    }
  }
  return 0;
}

/*
 * The same reduction for binary32 expert outputs ("MORI JIT v2", section 3.7:
 * combine reduces bf16 or fp32 rows and writes the same type): binary32 in,
 * binary32 accumulation from +0.0 in k order, then the binary32 bias
 * (fp32 [T, H] or NULL), binary32 out (no final rounding step).
 */
int oracle_combine_f32(const float *y, int32_t H, const float *topk_weights,
                       const float *bias, const int32_t *dst_slot, int32_t T, int32_t K,
                       int64_t capacity_rows, float *out) {
  if (T < 0 || K < 1 || H < 0) return -1;
  for (int32_t t = 0; t < T; ++t) {
    const int32_t *d = dst_slot + (int64_t)t * K;
    for (int32_t k = 0; k < K; ++k)
      if (d[k] >= capacity_rows) return -1;
    for (int32_t h = 0; h < H; ++h) {
      float acc = 0.0f;
      for (int32_t k = 0; k < K; ++k) {
        if (d[k] < 0) continue;
        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;
        float prod = w * y[(int64_t)d[k] * H + h];
        acc = acc + prod;
      }
      if (bias) acc = acc + bias[(int64_t)t * H + h];
      out[(int64_t)t * H + h] = acc;
    }
  }
  return 0;
}

/* Exposed for the tests that pin the rounding against hand-worked values. */
uint16_t oracle_f32_to_bf16(float f) { return float_to_bf16_bits_rne(f); }
float oracle_bf16_to_f32(uint16_t b) { return bf16_bits_to_float(b); }
