"""Seeded synthetic workloads for MoE layout / dispatch / combine.

This module only synthesises inputs (routing, router weights, activations,
fp8 scales, expert outputs). It holds none of the layout, dispatch or
combine arithmetic, so both the GPU path and the CPU oracle can consume its
arrays. Every array comes from ``np.random.default_rng([seed, stream])`` with
one stream per quantity: 0 routing, 1 router logits, 2 activations,
3 fp8 scales, 4 expert outputs, 5 masking. Casts to bf16 and fp8 e4m3fn go
through torch's CPU conversions (round to nearest even).

Workloads (sizes follow the pages: the MORI v2 default EpCfg shape and the
DeepEP dispatch_impl instance with hidden 7168, 256 experts, top-8 and an
expert alignment of 128):

=================  =====  ======  ====  ==  ===  =====  ===========================
name                T      H       E     K   A    dtype  routing
=================  =====  ======  ====  ==  ===  =====  ===========================
tiny                64     256     16    2   1    bf16   uniform distinct
mori_default        1024   7168    64    8   1    bf16   uniform distinct
decode_zipf         128    7168    256   8   1    bf16   Zipf(1.1) without replacement
prefill_aligned     4096   7168    256   8   128  bf16   uniform distinct
fp8_hot8            8192   7168    256   8   1    fp8    8 hot experts at 4x mean load
=================  =====  ======  ====  ==  ===  =====  ===========================
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16 = 0
FP32 = 1
FP8_E4M3 = 2
FP4X2 = 3

STREAM_ROUTING, STREAM_LOGITS, STREAM_X, STREAM_SCALES, STREAM_Y, STREAM_MASK = range(6)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int
    H: int
    E: int
    K: int
    A: int
    dtype: int
    routing: str
    capacity: int = 0  # 0 -> worst case T*K + E*(A-1)
    out_dtype: int = BF16  # element type of the expert outputs and the combined rows
    scales: bool = True    # fp8 / fp4x2: a scale row travels with each token

    @property
    def cap(self) -> int:
        return self.capacity or capacity_rows(self.T, self.K, self.E, self.A)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 64, 256, 16, 2, 1, BF16, "uniform"),
    "mori_default": Workload("mori_default", 2, 1024, 7168, 64, 8, 1, BF16, "uniform",
                             capacity=1024 * 8),
    "decode_zipf": Workload("decode_zipf", 3, 128, 7168, 256, 8, 1, BF16, "zipf"),
    "prefill_aligned": Workload("prefill_aligned", 4, 4096, 7168, 256, 8, 128, BF16, "uniform"),
    "fp8_hot8": Workload("fp8_hot8", 5, 8192, 7168, 256, 8, 1, FP8_E4M3, "hot8"),
}


# The same prefill shape with the other transport / reduction types: fp4x2 rows
# (3584 bytes = 7168 e2m1 values, 56 scales per token), binary32 expert
# outputs for combine, and binary32 throughout (rows and expert outputs); and
# a long prefill batch of 32768 tokens, whose x (470 MB) is larger than the
# 256 MB last-level cache.
EXTRA_WORKLOADS = {
    "prefill_fp4x2": Workload("prefill_fp4x2", 6, 4096, 3584, 256, 8, 128, FP4X2, "uniform"),
    "prefill_fp32_combine": Workload("prefill_fp32_combine", 7, 4096, 7168, 256, 8, 128, BF16,
                                     "uniform", out_dtype=FP32),
    "prefill_32k": Workload("prefill_32k", 8, 32768, 7168, 256, 8, 128, BF16, "uniform"),
    "prefill_fp32": Workload("prefill_fp32", 9, 4096, 7168, 256, 8, 128, FP32, "uniform",
                             out_dtype=FP32),
}


def capacity_rows(T: int, K: int, E: int, A: int) -> int:
    """Worst-case expand-buffer rows: every (t, k) real plus full padding per expert."""
    return T * K + E * (A - 1)


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------

def routing_uniform(g: np.random.Generator, T: int, E: int, K: int) -> np.ndarray:
    """K distinct experts per token, uniformly at random."""
    if T == 0:
        return np.zeros((0, K), np.int32)
    return np.argsort(g.random((T, E)), axis=1, kind="stable")[:, :K].astype(np.int32)


def routing_zipf(g: np.random.Generator, T: int, E: int, K: int, s: float = 1.1) -> np.ndarray:
    """K distinct experts per token from a Zipf(s) popularity, without replacement.

    Popularity of rank r (1-based) is proportional to r**-s; ranks map to
    expert ids through a seeded permutation. Sampling without replacement
    uses Gumbel-top-k on the log-popularity (Plackett-Luce).
    """
    ranks = np.arange(1, E + 1, dtype=np.float64)
    logp = -s * np.log(ranks)
    perm = g.permutation(E)
    gumbel = -np.log(-np.log(g.random((T, E))))
    top = np.argsort(-(logp[None, :] + gumbel), axis=1, kind="stable")[:, :K]
    return perm[top].astype(np.int32)


def routing_hot(g: np.random.Generator, T: int, E: int, K: int, n_hot: int = 8) -> np.ndarray:
    """n_hot seeded hot experts, each picked by a token with probability 1/n_hot.

    The remaining K - (hot picks) slots take distinct cold experts uniformly,
    then the order of the K entries is shuffled per token. With K = n_hot = 8
    each hot expert's expected load is T/8, four times the mean T*K/E at E=256.
    """
    hot = g.choice(E, n_hot, replace=False)
    cold = np.setdiff1d(np.arange(E), hot)
    pick = g.random((T, n_hot)) < (1.0 / n_hot)
    cold_order = np.argsort(g.random((T, cold.size)), axis=1, kind="stable")
    out = np.empty((T, K), np.int32)
    for t in range(T):
        h = hot[pick[t]][:K]
        c = cold[cold_order[t, :K - h.size]]
        row = np.concatenate([h, c])
        g.shuffle(row)
        out[t] = row
    return out


def make_routing(routing: str, seed: int, T: int, E: int, K: int) -> np.ndarray:
    g = rng(seed, STREAM_ROUTING)
    if routing == "uniform":
        return routing_uniform(g, T, E, K)
    if routing == "zipf":
        return routing_zipf(g, T, E, K)
    if routing == "hot8":
        return routing_hot(g, T, E, K)
    raise ValueError(f"unknown routing {routing!r}")


def mask_entries(topk_idx: np.ndarray, seed: int, frac: float) -> np.ndarray:
    """Copy of topk_idx with a seeded fraction of entries set to -1 (masked)."""
    g = rng(seed, STREAM_MASK)
    out = topk_idx.copy()
    out[g.random(out.shape) < frac] = -1
    return out


# --------------------------------------------------------------------------
# Values
# --------------------------------------------------------------------------

def router_weights(seed: int, T: int, K: int) -> np.ndarray:
    """fp32 softmax over the K chosen experts of N(0, 1) logits."""
    logits = rng(seed, STREAM_LOGITS).standard_normal((T, K))
    if T == 0:
        return np.zeros((0, K), np.float32)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def _to_bf16_bits(a32: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def normal_bf16(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """N(0, 1) values rounded to bf16, returned as uint16 bit patterns."""
    g = rng(seed, stream)
    out = np.empty((rows, cols), np.uint16)
    step = max(1, (1 << 24) // max(cols, 1))
    for r0 in range(0, rows, step):  # bounded temporaries for the big buffers
        r1 = min(rows, r0 + step)
        out[r0:r1] = _to_bf16_bits(g.standard_normal((r1 - r0, cols), dtype=np.float32))
    return out


def normal_f32(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """N(0, 1) binary32 values."""
    return rng(seed, stream).standard_normal((rows, cols), dtype=np.float32)


def fp4x2_rows(seed: int, T: int, H_bytes: int):
    """Packed e2m1 pairs (any byte is a valid pair of codes) and fp32 scales.

    One scale per 128 values (64 bytes), s ~ U[0.01, 1]. Returns (uint8 [T, H_bytes],
    float32 [T, 2*H_bytes/128]).
    """
    q = rng(seed, STREAM_X).integers(0, 256, (T, H_bytes), dtype=np.uint8)
    S = max(1, (2 * H_bytes) // 128)
    s = rng(seed, STREAM_SCALES).uniform(0.01, 1.0, (T, S)).astype(np.float32)
    return q, s


def fp8_rows(seed: int, T: int, H: int):
    """e4m3fn activations with one fp32 scale per 128-channel block.

    x ~ N(0, 1), s ~ U[0.01, 1] per (token, block), q = e4m3fn(clamp(x / s, +-448)).
    Returns (q as uint8 [T, H], scales float32 [T, H/128]).
    """
    import torch
    assert H % 128 == 0
    S = H // 128
    x = rng(seed, STREAM_X).standard_normal((T, H), dtype=np.float32)
    s = rng(seed, STREAM_SCALES).uniform(0.01, 1.0, (T, S)).astype(np.float32)
    v = (x.reshape(T, S, 128) / s[:, :, None]).reshape(T, H)
    v = np.clip(v, -448.0, 448.0)
    q = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, s


@dataclass
class Case:
    """One synthetic input set. Byte arrays are numpy, host resident."""
    w: Workload
    topk_idx: np.ndarray            # int32 [T, K]
    topk_weights: np.ndarray        # float32 [T, K]
    x: np.ndarray                   # bf16 bits uint16, fp32, e4m3 or packed e2m1 bytes [T, H]
    x_scales: Optional[np.ndarray]  # float32 [T, values/128] for fp8 / fp4x2, else None
    y: Optional[np.ndarray] = None  # expert outputs [cap, H]: bf16 bits uint16 or fp32
    extra: dict = field(default_factory=dict)


def make_case(w: Workload, with_y: bool = True, mask_frac: float = 0.0) -> Case:
    idx = make_routing(w.routing, w.seed, w.T, w.E, w.K)
    if mask_frac > 0:
        idx = mask_entries(idx, w.seed, mask_frac)
    wts = router_weights(w.seed, w.T, w.K)
    if w.dtype == FP8_E4M3:
        x, xs = fp8_rows(w.seed, w.T, w.H)
    elif w.dtype == FP4X2:
        x, xs = fp4x2_rows(w.seed, w.T, w.H)
    elif w.dtype == BF16:
        x, xs = normal_bf16(w.seed, STREAM_X, w.T, w.H), None
    elif w.dtype == FP32:
        x, xs = normal_f32(w.seed, STREAM_X, w.T, w.H), None
    else:
        raise ValueError(f"unknown dtype {w.dtype}")
    if not w.scales:
        xs = None
    y = None
    if with_y:
        H_out = 2 * w.H if w.dtype == FP4X2 else w.H  # combine sees one value per element
        y = (normal_bf16(w.seed, STREAM_Y, w.cap, H_out) if w.out_dtype == BF16
             else normal_f32(w.seed, STREAM_Y, w.cap, H_out))
    return Case(w, idx, wts, x, xs, y)


def custom(name: str, seed: int, T: int, H: int, E: int, K: int, A: int = 1,
           dtype: int = BF16, routing: str = "uniform", capacity: int = 0,
           out_dtype: int = BF16, scales: bool = True) -> Workload:
    """A workload of arbitrary shape (for edge cases and ragged tails)."""
    return Workload(name, seed, T, H, E, K, A, dtype, routing, capacity, out_dtype, scales)
