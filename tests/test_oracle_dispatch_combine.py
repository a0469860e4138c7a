"""Pins for the oracle's dispatch (byte permute-copy) and combine (weighted gather-reduce).

Sources: MORI JIT v2 page, section 3.7 (dispatch moves payload bytes only,
fp8 rows arrive quantised, combine reduces bf16); DeepEP overall-architecture
page, dispatch / combine data-flow figure (copy epilogue with token data and
scale factors; reduce epilogue weighted by topk_weights).
"""
import json
import os

import numpy as np
import pytest

from combine_ep_layout_amd import inputs as I
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex(v):
    return int(v, 16)


def test_rounding_hand_worked(oracle_mod):
    data = json.load(open(os.path.join(GOLDEN, "combine_worked_examples.json")))
    assert data["source"]
    for r in data["rounding"]:
        f = np.array([_hex(r["f32_hex"])], np.uint32).view(np.float32)[0]
        assert oracle_mod.f32_to_bf16(f) == _hex(r["bf16_hex"]), r["note"]
    # NaN stays NaN (quiet), sign kept
    for nan_bits in (0x7FC00000, 0x7F800001, 0xFFC00123, 0x7FFFFFFF, 0xFFFFFFFF):
        f = np.array([nan_bits], np.uint32).view(np.float32)[0]
        b = oracle_mod.f32_to_bf16(f)
        assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0 and (b & 0x0040)
        assert (b >> 15) == (nan_bits >> 31)


def test_combine_hand_worked(oracle_mod):
    data = json.load(open(os.path.join(GOLDEN, "combine_worked_examples.json")))
    for c in data["combine"]:
        y = np.array([[_hex(v) for v in row] for row in c["y_rows_hex"]], np.uint16)
        dst = np.array(c["dst_slot"], np.int32)
        w = None if c["topk_weights"] is None else np.array(c["topk_weights"], np.float32)
        out = oracle_mod.combine(y, dst, w)
        exp = np.array([[_hex(v) for v in row] for row in c["out_hex"]], np.uint16)
        assert np.array_equal(out, exp), c["name"]


def _layout(oracle_mod, w):
    idx = I.make_routing(w.routing, w.seed, w.T, w.E, w.K)
    return idx, oracle_mod.layout(idx, w.E, w.A)


CASES = [I.custom("c1", 11, 37, 64, 8, 2, 1), I.custom("c2", 12, 100, 256, 16, 4, 8),
         I.custom("c3", 13, 65, 512, 64, 8, 16), I.custom("c4", 14, 9, 128, 4, 1, 1),
         I.custom("c5", 15, 50, 384, 32, 6, 4)]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_dispatch_bf16_bytes(oracle_mod, w):
    case = I.make_case(w, with_y=False)
    _, lay = _layout(oracle_mod, w)
    before = np.random.default_rng(0).integers(0, 256, (w.cap, w.H * 2), dtype=np.uint8)
    X, _, Xw = oracle_mod.dispatch(case.x, lay["dst_slot"], w.cap, topk_weights=case.topk_weights,
                                   expand_x=before.copy())
    pins.check_dispatch(case.x.view(np.uint8).reshape(w.T, -1), lay["dst_slot"], before, X)
    # the same through numpy fancy indexing
    assert np.array_equal(X.reshape(w.cap, -1)[lay["dst_slot"].ravel()],
                          np.repeat(case.x.view(np.uint8).reshape(w.T, -1), w.K, axis=0))
    assert np.array_equal(Xw[lay["dst_slot"].ravel()], case.topk_weights.ravel())


def test_dispatch_fp8_with_scales(oracle_mod):
    w = I.custom("fp8", 21, 70, 512, 32, 4, 2, I.FP8_E4M3, "hot8")
    case = I.make_case(w, with_y=False)
    assert case.x.dtype == np.uint8 and case.x_scales.shape == (70, 4)
    _, lay = _layout(oracle_mod, w)
    bx = np.full((w.cap, w.H), 0xAB, np.uint8)
    bs = np.full((w.cap, 4), -7.0, np.float32)
    X, Xs, _ = oracle_mod.dispatch(case.x, lay["dst_slot"], w.cap, x_scales=case.x_scales,
                                   expand_x=bx.copy(), expand_scales=bs.copy())
    pins.check_dispatch(case.x, lay["dst_slot"], bx, X)
    pins.check_dispatch(case.x_scales.view(np.uint8).reshape(w.T, -1), lay["dst_slot"],
                        bs.view(np.uint8).reshape(w.cap, -1), Xs.view(np.uint8).reshape(w.cap, -1))


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_error_bound(oracle_mod, w, weighted):
    case = I.make_case(w)
    _, lay = _layout(oracle_mod, w)
    wts = case.topk_weights if weighted else None
    out = oracle_mod.combine(case.y, lay["dst_slot"], wts)
    pins.check_combine_bound(case.y, lay["dst_slot"], wts, out)


def test_combine_error_bound_heavy_cancellation(oracle_mod):
    # pairs of nearly opposite rows make the result tiny relative to the terms
    w = I.custom("cancel", 31, 64, 256, 8, 4, 1)
    case = I.make_case(w)
    _, lay = _layout(oracle_mod, w)
    y = case.y.copy()
    dst = lay["dst_slot"]
    y[dst[:, 1]] = y[dst[:, 0]] ^ np.uint16(0x8000)   # row for k=1 is minus row for k=0
    wts = np.full((w.T, w.K), 0.25, np.float32)
    wts[:, 1] = np.float32(0.25) * np.float32(1 + 2 ** -20)
    out = oracle_mod.combine(y, dst, wts)
    pins.check_combine_bound(y, dst, wts, out)


def test_combine_k1_unit_weight_is_a_gather(oracle_mod):
    w = I.custom("k1", 41, 90, 256, 12, 1, 4)
    case = I.make_case(w)
    _, lay = _layout(oracle_mod, w)
    out = oracle_mod.combine(case.y, lay["dst_slot"], np.ones((w.T, 1), np.float32))
    assert np.array_equal(out, case.y[lay["dst_slot"][:, 0]])
    out = oracle_mod.combine(case.y, lay["dst_slot"], None)
    assert np.array_equal(out, case.y[lay["dst_slot"][:, 0]])


@pytest.mark.parametrize("name", ["tiny", "decode_zipf"])
def test_identity_expert_round_trip_bf16(oracle_mod, name):
    """dispatch -> identity expert -> combine with softmax weights returns x exactly.

    The binary32 sum differs from x by at most about K * 2^-24 |x| plus
    |1 - sum w| |x|, far below half a bf16 spacing (at least 2^-9 |x|).
    """
    w = I.WORKLOADS[name]
    case = I.make_case(w, with_y=False)
    _, lay = _layout(oracle_mod, w)
    X, _, _ = oracle_mod.dispatch(case.x, lay["dst_slot"], w.cap)
    out = oracle_mod.combine(X.view(np.uint16).reshape(w.cap, w.H), lay["dst_slot"], case.topk_weights)
    assert np.array_equal(out, case.x)


def test_identity_expert_round_trip_fp8(oracle_mod):
    """fp8 dispatch, the expert dequantises bf16(f32(q) * s), combine returns that exactly."""
    import torch
    w = I.custom("fp8rt", 51, 96, 512, 64, 8, 1, I.FP8_E4M3, "hot8")
    case = I.make_case(w, with_y=False)
    _, lay = _layout(oracle_mod, w)
    X, Xs, _ = oracle_mod.dispatch(case.x, lay["dst_slot"], w.cap, x_scales=case.x_scales)
    S = w.H // 128

    def dequant(q, s):
        qf = torch.from_numpy(q.copy()).view(torch.float8_e4m3fn).float().reshape(-1, S, 128)
        return (qf * torch.from_numpy(s.copy()).reshape(-1, S, 1)).reshape(-1, w.H) \
            .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    y = dequant(X, Xs.view(np.float32).reshape(w.cap, S))
    out = oracle_mod.combine(y, lay["dst_slot"], case.topk_weights)
    # e4m3 0x80 is -0: the sum starts at +0.0, so -0 comes back as +0 (equal values)
    assert pins.bf16_ulp_distance(out, dequant(case.x, case.x_scales)).max() == 0


def test_combine_masked_entries_are_skipped(oracle_mod):
    w = I.custom("mask", 61, 40, 128, 8, 4, 2)
    case = I.make_case(w, mask_frac=0.3)
    lay = oracle_mod.layout(case.topk_idx, w.E, w.A)
    out = oracle_mod.combine(case.y, lay["dst_slot"], case.topk_weights)
    pins.check_combine_bound(case.y, lay["dst_slot"], case.topk_weights, out)
    dead = (lay["dst_slot"] < 0).all(axis=1)
    assert np.all(out[dead] == 0)  # +0.0 for tokens with nothing routed


def test_ulp_distance_helper():
    a = np.array([0x3F80, 0x8000, 0x0000, 0xBF80, 0x0001], np.uint16)
    b = np.array([0x3F81, 0x0000, 0x8001, 0xBF81, 0x8001], np.uint16)
    assert pins.bf16_ulp_distance(a, b).tolist() == [1, 0, 1, 1, 2]


def test_combine_f32_hand_worked(oracle_mod):
    data = json.load(open(os.path.join(GOLDEN, "combine_worked_examples.json")))
    for c in data["combine_f32"]:
        y = np.array(c["y_rows"], np.float32)
        out = oracle_mod.combine_f32(y, np.array(c["dst_slot"], np.int32),
                                     np.array(c["topk_weights"], np.float32))
        exp = np.array(c["out"], np.float32)
        assert np.array_equal(out.view(np.uint32), exp.view(np.uint32)), c["name"]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
@pytest.mark.parametrize("weighted", [True, False])
def test_combine_f32_error_bound(oracle_mod, w, weighted):
    g = np.random.default_rng([w.seed, 7])
    y = g.standard_normal((w.cap, w.H)).astype(np.float32)
    _, lay = _layout(oracle_mod, w)
    wts = I.router_weights(w.seed, w.T, w.K) if weighted else None
    out = oracle_mod.combine_f32(y, lay["dst_slot"], wts)
    pins.check_combine_bound_f32(y, lay["dst_slot"], wts, out)


def test_combine_f32_k1_and_masking(oracle_mod):
    w = I.custom("f32k1", 43, 70, 256, 12, 1, 2)
    _, lay = _layout(oracle_mod, w)
    y = np.random.default_rng(3).standard_normal((w.cap, w.H)).astype(np.float32)
    out = oracle_mod.combine_f32(y, lay["dst_slot"], None)
    assert np.array_equal(out, y[lay["dst_slot"][:, 0]])
    dst = lay["dst_slot"].copy()
    dst[::3] = -1
    out = oracle_mod.combine_f32(y, dst, np.ones((w.T, 1), np.float32))
    assert np.all(out[::3].view(np.uint32) == 0) and np.array_equal(out[1::3], y[dst[1::3, 0]])


def test_combine_bias_hand_worked(oracle_mod):
    data = json.load(open(os.path.join(GOLDEN, "combine_worked_examples.json")))
    for c in data["combine_bias"]:
        y = np.array([[_hex(v) for v in row] for row in c["y_rows_hex"]], np.uint16)
        b = np.array([[_hex(v) for v in row] for row in c["bias_hex"]], np.uint16)
        out = oracle_mod.combine(y, np.array(c["dst_slot"], np.int32), None, b)
        assert np.array_equal(out, np.array([[_hex(v) for v in r] for r in c["out_hex"]], np.uint16))
    for c in data["combine_f32_bias"]:
        out = oracle_mod.combine_f32(np.array(c["y_rows"], np.float32), np.array(c["dst_slot"], np.int32),
                                     np.array(c["topk_weights"], np.float32), np.array(c["bias"], np.float32))
        assert np.array_equal(out.view(np.uint32), np.array(c["out"], np.float32).view(np.uint32))


@pytest.mark.parametrize("w", CASES[:3], ids=lambda w: w.name)
def test_combine_bias_error_bound(oracle_mod, w):
    case = I.make_case(w)
    _, lay = _layout(oracle_mod, w)
    bias = I.normal_bf16(w.seed, 9, w.T, w.H)
    out = oracle_mod.combine(case.y, lay["dst_slot"], case.topk_weights, bias)
    pins.check_combine_bound(case.y, lay["dst_slot"], case.topk_weights, out, bias)
    yf = np.random.default_rng(2).standard_normal((w.cap, w.H)).astype(np.float32)
    bf = np.random.default_rng(3).standard_normal((w.T, w.H)).astype(np.float32)
    out = oracle_mod.combine_f32(yf, lay["dst_slot"], case.topk_weights, bf)
    pins.check_combine_bound_f32(yf, lay["dst_slot"], case.topk_weights, out, bf)


@pytest.mark.parametrize("w", [I.custom("zp1", 71, 300, 256, 16, 4, 8), I.custom("zp2", 72, 40, 512, 64, 2, 32),
                               I.custom("zp3", 73, 100, 256, 8, 8, 1)], ids=lambda w: w.name)
def test_zero_padding(oracle_mod, w):
    """Exactly the padding rows [off[e] + count[e], off[e+1]) become zero (counts and offsets
    from the library route, not the oracle); every other row keeps its bytes."""
    idx = I.make_routing(w.routing, w.seed, w.T, w.E, w.K)
    counts, offsets, _, _ = pins.layout_by_argsort(idx, w.E, w.A)
    g = np.random.default_rng(w.seed)
    X = g.integers(1, 256, (w.cap, w.H), dtype=np.uint8)
    S = g.integers(1, 256, (w.cap, 16), dtype=np.uint8)
    Wt = g.random(w.cap).astype(np.float32) + 1
    before = (X.copy(), S.copy(), Wt.copy())
    oracle_mod.zero_padding(X, counts, offsets, S, Wt)
    pad = np.zeros(w.cap, bool)
    for e in range(w.E):
        pad[offsets[e] + counts[e]:offsets[e + 1]] = True
    assert pad.sum() == offsets[-1] - counts.sum()
    for a, b in zip((X, S, Wt), before):
        assert np.all(a[pad] == 0) and np.array_equal(a[~pad], b[~pad])
