"""Independent checks that pin the oracle (and, by extension, the GPU path).

Nothing here calls the oracle. Each check derives the expected result by a
different route than the oracle's loops: brute force over all pairs, numpy
library routines (bincount, stable argsort, fancy indexing), invariants that
any correct layout satisfies, and a float64 evaluation of the weighted sum
with a rigorous binary32 error bound. The mutation test plants mistakes in a
copy of the oracle and requires every one of them to trip at least one check.
"""
import numpy as np

U32 = 2.0 ** -24  # binary32 unit roundoff


# --------------------------------------------------------------------------
# Layout
# --------------------------------------------------------------------------

def _valid(idx, E):
    return (idx >= 0) & (idx < E)


def layout_bruteforce(idx, E, A):
    """Definition-by-enumeration; O((T*K)^2), for tiny inputs only."""
    T, K = idx.shape
    flat = idx.ravel()
    n = flat.size
    counts = np.array([sum(1 for i in range(n) if flat[i] == e) for e in range(E)], np.int64)
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + int(np.ceil(counts[e] / A)) * A if counts[e] else offsets[-1])
    dst = np.full(n, -1, np.int64)
    for i in range(n):
        e = flat[i]
        if 0 <= e < E:
            before = sum(1 for j in range(i) if flat[j] == e)
            dst[i] = offsets[e] + before
    dst = dst.reshape(T, K)
    rows = [[t, 0] + list(dst[t]) for t in range(T) if (dst[t] >= 0).any()]
    return counts, np.array(offsets), dst, rows


def layout_by_argsort(idx, E, A):
    """Library route: bincount for counts, stable argsort for ranks."""
    T, K = idx.shape
    flat = idx.ravel().astype(np.int64)
    v = _valid(flat, E)
    counts = np.bincount(flat[v], minlength=E)
    padded = -(-counts // A) * A
    offsets = np.concatenate([[0], np.cumsum(padded)])
    key = np.where(v, flat, E)                      # masked entries sort last
    order = np.argsort(key, kind="stable")          # token-major within each expert
    sorted_key = key[order]
    first = np.searchsorted(sorted_key, sorted_key, side="left")
    rank = np.empty_like(order)
    rank[order] = np.arange(order.size) - first
    dst = np.where(v, offsets[np.minimum(key, E - 1)] + rank, -1) if E > 0 else np.full_like(flat, -1)
    dst = dst.reshape(T, K)
    has = (dst >= 0).any(axis=1)
    toks = np.nonzero(has)[0]
    meta = np.concatenate([toks[:, None], np.zeros((toks.size, 1), np.int64), dst[toks]], axis=1) \
        if toks.size else np.zeros((0, K + 2), np.int64)
    return counts, offsets, dst, meta


def check_layout_invariants(idx, E, A, res):
    T, K = idx.shape
    counts, offsets, dst = res["counts"].astype(np.int64), res["offsets"].astype(np.int64), \
        res["dst_slot"].astype(np.int64)
    v = _valid(idx, E)
    n_valid = int(v.sum())
    assert counts.sum() == n_valid, "counts must sum to the number of unmasked entries"
    assert offsets[0] == 0
    assert np.all(offsets % A == 0), "every segment starts on an alignment boundary"
    seg = np.diff(offsets)
    assert np.all(seg >= counts) and np.all(seg - counts < A), "segment = count padded up to A"
    assert np.all((counts == 0) == (seg == 0)), "an empty expert gets no rows"
    assert n_valid <= offsets[-1] <= T * K + E * (A - 1), "capacity bound"
    assert np.all(dst[~v] == -1), "masked entries have no slot"
    for e in range(E):
        mine = dst[idx == e]  # token-major order
        local = mine - offsets[e]
        assert np.array_equal(local, np.arange(counts[e])), \
            f"expert {e}: slots must be offset + 0..count-1 in token-major order"
    has = v.any(axis=1)
    assert res["num_recv"] == int(has.sum())
    meta = np.asarray(res["recv_src_metadata"], np.int64)
    assert meta.shape == (int(has.sum()), K + 2)
    assert np.array_equal(meta[:, 0], np.nonzero(has)[0])
    assert np.all(meta[:, 1] == 0)
    assert np.array_equal(meta[:, 2:], dst[has])


def check_layout_matches(res, counts, offsets, dst, meta):
    assert np.array_equal(res["counts"], counts), "counts"
    assert np.array_equal(res["offsets"], offsets), "offsets"
    assert np.array_equal(res["dst_slot"], dst), "dst_slot"
    assert np.array_equal(np.asarray(res["recv_src_metadata"]).reshape(-1, dst.shape[1] + 2),
                          np.asarray(meta).reshape(-1, dst.shape[1] + 2)), "recv_src_metadata"


# --------------------------------------------------------------------------
# Dispatch
# --------------------------------------------------------------------------

def check_dispatch(x_rows, dst, before, after):
    """x_rows [T, B] bytes; before/after [cap, B]: expand buffer around the call."""
    T, K = dst.shape
    v = dst >= 0
    d = dst[v]
    t = np.repeat(np.arange(T), K).reshape(T, K)[v]
    assert np.unique(d).size == d.size, "each real row is written exactly once"
    assert np.array_equal(after[d], x_rows[t]), "expand row dst[t,k] holds x[t]"
    untouched = np.ones(after.shape[0], bool)
    untouched[d] = False
    assert np.array_equal(after[untouched], before[untouched]), "padding rows are not written"


# --------------------------------------------------------------------------
# Combine
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(x64):
    """Spacing of bf16 numbers at |x| (8 significant bits, binary32 exponent range)."""
    a = np.abs(x64)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, 2.0 ** (e - 7), 2.0 ** -133)


def combine_exact(y_bits, dst, w, bias_bits=None):
    """float64 value of sum_k w[t,k] * y[dst[t,k]] (+ bias) over unmasked k, and sum |terms|."""
    T, K = dst.shape
    yf = bf16_bits_to_f64(y_bits)
    v = dst >= 0
    rows = yf[np.where(v, dst, 0)] * v[..., None]
    wf = np.ones((T, K)) if w is None else np.asarray(w, np.float32).astype(np.float64)
    p = rows * wf[..., None]
    exact, absum = p.sum(axis=1), np.abs(p).sum(axis=1)
    if bias_bits is not None:
        b = bf16_bits_to_f64(bias_bits)
        exact, absum = exact + b, absum + np.abs(b)
    return exact, absum


def check_combine_bound(y_bits, dst, w, out_bits, bias_bits=None):
    """|out - exact| <= gamma_n * sum|terms| + half a bf16 ulp of out.

    gamma_n = n u / (1 - n u) bounds n binary32 roundings per term (one
    product, at most K-1 sums, one more for a bias) in a recursive sum; the
    final bf16 rounding to nearest adds at most half a spacing of the result.
    """
    T, K = dst.shape
    exact, absum = combine_exact(y_bits, dst, w, bias_bits)
    out = bf16_bits_to_f64(out_bits)
    n = K + (bias_bits is not None)
    gamma = n * U32 / (1 - n * U32)
    bound = gamma * absum + 0.5 * bf16_ulp(out) + 2.0 ** -50 * absum
    err = np.abs(out - exact)
    bad = err > bound
    assert not bad.any(), f"{int(bad.sum())} outputs exceed the error bound, worst {err[bad].max()}"


def check_combine_bound_f32(y, dst, w, out, bias=None):
    """Binary32 output: |out - exact| <= gamma_n * sum|terms| (no final rounding step)."""
    T, K = dst.shape
    yf = np.asarray(y, np.float32).astype(np.float64)
    v = dst >= 0
    rows = yf[np.where(v, dst, 0)] * v[..., None]
    wf = np.ones((T, K)) if w is None else np.asarray(w, np.float32).astype(np.float64)
    p = rows * wf[..., None]
    exact, absum = p.sum(axis=1), np.abs(p).sum(axis=1)
    if bias is not None:
        b = np.asarray(bias, np.float32).astype(np.float64)
        exact, absum = exact + b, absum + np.abs(b)
    n = K + (bias is not None)
    gamma = n * U32 / (1 - n * U32)
    err = np.abs(np.asarray(out, np.float64) - exact)
    bad = err > gamma * absum + 2.0 ** -50 * absum + 2.0 ** -149
    assert not bad.any(), f"{int(bad.sum())} outputs exceed the binary32 error bound"


def bf16_ulp_distance(a_bits, b_bits):
    """Distance in units of bf16 spacing between two bf16 bit arrays (ordered integers)."""
    def ordered(b):
        b = np.asarray(b, np.uint16).astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


# --------------------------------------------------------------------------
# Non-expand (one row per received token)
# --------------------------------------------------------------------------

def check_dispatch_compact(x_rows, topk_idx, dst, meta, num_recv, recv_x, recv_idx, w=None, recv_w=None):
    """recv row i holds token meta[i, 0]; ids of masked entries read -1."""
    toks = np.asarray(meta)[:num_recv, 0]
    assert np.array_equal(recv_x[:num_recv], x_rows[toks]), "recv_x[i] = x[meta[i, 0]]"
    masked = np.where(dst >= 0, topk_idx, -1)
    assert np.array_equal(recv_idx[:num_recv], masked[toks]), "recv_topk_idx"
    if w is not None:
        assert np.array_equal(recv_w[:num_recv], np.asarray(w)[toks]), "recv_topk_weights"


def check_combine_compact(y_bits, dst, meta, num_recv, out_bits, bias_bits=None):
    """out[t] = y[row of t] (+ bias) with one rounding; +0 (+ bias) for unreceived tokens."""
    T = dst.shape[0]
    row_of = np.full(T, -1)
    row_of[np.asarray(meta)[:num_recv, 0]] = np.arange(num_recv)
    recv = (dst >= 0).any(axis=1)
    assert np.array_equal(recv, row_of >= 0), "exactly the tokens with an unmasked entry are received"
    yv = np.where(recv[:, None], bf16_bits_to_f64(np.asarray(y_bits)[np.maximum(row_of, 0)]), 0.0)
    if bias_bits is None:
        exp = np.where(recv[:, None], np.asarray(y_bits)[np.maximum(row_of, 0)], 0).astype(np.uint16)
        assert np.array_equal(out_bits, exp), "without a bias rows come back bit for bit"
        return
    exact = yv + bf16_bits_to_f64(bias_bits)
    out = bf16_bits_to_f64(out_bits)
    # two binary32 roundings of a sum of two bf16 values (the first is exact) then bf16 rounding
    bound = 0.5 * bf16_ulp(out) + U32 * np.abs(exact)
    assert np.all(np.abs(out - exact) <= bound), "bias add outside half a bf16 ulp"


def check_combine_compact_f32(y, dst, meta, num_recv, out, bias=None):
    """Binary32 rows: out[t] = y[row of t] (+ bias) with one binary32 rounding;
    +0 (+ bias) for unreceived tokens. The sum is evaluated in float64, where
    the sum of two binary32 values of similar size is exact."""
    T = dst.shape[0]
    row_of = np.full(T, -1)
    row_of[np.asarray(meta)[:num_recv, 0]] = np.arange(num_recv)
    recv = (dst >= 0).any(axis=1)
    assert np.array_equal(recv, row_of >= 0), "exactly the tokens with an unmasked entry are received"
    y = np.asarray(y, np.float32)
    got = np.where(recv[:, None], y[np.maximum(row_of, 0)], np.float32(0.0)).astype(np.float32)
    if bias is None:
        assert np.array_equal(out.view(np.uint32), got.view(np.uint32)), \
            "without a bias rows come back bit for bit (+0 for unreceived tokens)"
        return
    exact = got.astype(np.float64) + np.asarray(bias, np.float64)
    ulp = np.spacing(np.abs(out).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(out.astype(np.float64) - exact) <= 0.5 * ulp + 2.0 ** -53 * np.abs(exact)), \
        "bias add outside half a binary32 ulp"


# --------------------------------------------------------------------------
# Dispatch plan
# --------------------------------------------------------------------------

def dispatch_plan(dst, E, K):
    """The dispatch plan ep_layout writes, as include/ep_mi355x.h defines it,
    computed from the oracle's slots: per tile of floor(W / K) tokens (W =
    1024, 512 or 256 for E up to 256, 512, 1024), the unmasked entries by
    ascending slot as (entry, slot), then (-1, -1) once per masked entry. The
    plan is the library's write-order aid, not part of the pages' method."""
    T = dst.shape[0]
    W = 1024 if E <= 256 else (512 if E <= 512 else 256)
    tokens = W // K
    flat = dst.reshape(-1)
    out = np.full((T * K, 2), -1, np.int32)
    for t0 in range(0, T, tokens):
        lo, hi = t0 * K, min(T, t0 + tokens) * K
        seg = flat[lo:hi]
        valid = np.nonzero(seg >= 0)[0]
        order = valid[np.argsort(seg[valid], kind="stable")]
        out[lo:lo + order.size, 0] = lo + order
        out[lo:lo + order.size, 1] = seg[order]
    return out
