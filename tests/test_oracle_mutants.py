"""The pins must catch plausible mistakes in the oracle.

Each case copies ep_oracle.c, plants one mistake by text substitution (a
dropped term, a wrong sign, a wrong index, a transposed operand, a wrong
rounding, a wrong loop order ...), builds the copy with gcc and runs the
pin suite against it. Every planted mistake must trip at least one pin.
This runs on the CPU only; nothing here touches the GPU.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from combine_ep_layout_amd import inputs as I
from tests import pins

MUTANTS = {
    "floor_instead_of_ceil": ("((counts[e] + A - 1) / A) * A", "(counts[e] / A) * A"),
    "no_alignment": ("int32_t padded = ((counts[e] + A - 1) / A) * A;", "int32_t padded = counts[e];"),
    "inclusive_cursor": ("cursor[e] = offsets[e];", "cursor[e] = offsets[e] + 1;"),
    "inclusive_prefix_cursor": ("cursor[e] = offsets[e];", "cursor[e] = offsets[e + 1];"),
    "k_major_order": ("for (int32_t t = 0; t < T; ++t) {\n    for (int32_t k = 0; k < K; ++k) {\n      int64_t i = (int64_t)t * K + k;",
                      "for (int32_t k = 0; k < K; ++k) {\n    for (int32_t t = 0; t < T; ++t) {\n      int64_t i = (int64_t)t * K + k;"),
    "count_set_not_add": ("if (e >= 0 && e < E) counts[e] += 1;", "if (e >= 0 && e < E) counts[e] = 1;"),
    "masked_token_kept": ("    if (!any) continue;\n", ""),
    "meta_rank_is_token": ("row[1] = 0; /* source rank: a world of one */", "row[1] = t;"),
    "meta_slot_shift": ("row[2 + k] = dst_slot[(int64_t)t * K + k];", "row[2 + k] = dst_slot[(int64_t)t * K + (K - 1 - k)];"),
    "meta_token_index": ("row[0] = t;", "row[0] = i;"),
    "dispatch_wrong_token": ("x + (int64_t)t * row_bytes", "x + (int64_t)(T - 1 - t) * row_bytes", 0),
    "dispatch_scales_dropped": ("      if (x_scales && expand_scales)\n", "      if (0)\n"),
    "dispatch_weight_k0": ("expand_weights[d] = topk_weights[(int64_t)t * K + k];", "expand_weights[d] = topk_weights[(int64_t)t * K];"),
    "combine_truncate": ("u += 0x7fffu + lsb;", "u += 0u * lsb;"),
    "combine_round_half_up": ("u += 0x7fffu + lsb;", "u += 0x8000u + 0u * lsb;"),
    "combine_drop_last_term": ("      for (int32_t k = 0; k < K; ++k) {\n        if (d[k] < 0) continue;",
                               "      for (int32_t k = 0; k < K - 1; ++k) {\n        if (d[k] < 0) continue;", 0),
    "combine_wrong_sign": ("acc = acc + prod;", "acc = acc - prod;", 0),
    "combine_transposed_weight": ("float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;",
                                  "float w = topk_weights ? topk_weights[(int64_t)k * T + t] : 1.0f;", 0),
    "combine_row_k0": ("float v = bf16_bits_to_float(y[(int64_t)d[k] * H + h]);",
                       "float v = bf16_bits_to_float(y[(int64_t)d[0] * H + h]);"),
    "combine_unweighted_default_zero": ("topk_weights[(int64_t)t * K + k] : 1.0f;", "topk_weights[(int64_t)t * K + k] : 0.5f;", 0),
    "combine_nan_guard_dropped": ("  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)\n"
                                  "    return (uint16_t)((u >> 16) | 0x0040u);\n", ""),
    "combine_fp16_style_bias": ("uint32_t lsb = (u >> 16) & 1u;", "uint32_t lsb = (u >> 15) & 1u;"),
    "combine_f32_wrong_sign": ("        float prod = w * y[(int64_t)d[k] * H + h];\n        acc = acc + prod;",
                               "        float prod = w * y[(int64_t)d[k] * H + h];\n        acc = acc - prod;"),
    "combine_f32_row_k0": ("float prod = w * y[(int64_t)d[k] * H + h];", "float prod = w * y[(int64_t)d[0] * H + h];"),
    "combine_f32_drop_first_term": ("      for (int32_t k = 0; k < K; ++k) {\n        if (d[k] < 0) continue;\n        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;\n        float prod",
                                    "      for (int32_t k = 1; k < K; ++k) {\n        if (d[k] < 0) continue;\n        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;\n        float prod"),
    "combine_bias_dropped": ("      if (bias) acc = acc + bf16_bits_to_float(bias[(int64_t)t * H + h]);\n", ""),
    "combine_bias_twice": ("float acc = 0.0f;", "float acc = bias ? bf16_bits_to_float(bias[(int64_t)t * H + h]) : 0.0f;", 0),
    "combine_f32_bias_dropped": ("      if (bias) acc = acc + bias[(int64_t)t * H + h];\n", ""),
    "combine_f32_bias_first": ("float acc = 0.0f;", "float acc = bias ? bias[(int64_t)t * H + h] : 0.0f;", 1),
    "zero_padding_from_segment_start": ("for (int64_t r = (int64_t)offsets[e] + counts[e]; r < offsets[e + 1]; ++r) {",
                                        "for (int64_t r = (int64_t)offsets[e]; r < offsets[e + 1]; ++r) {"),
    "zero_padding_one_short": ("for (int64_t r = (int64_t)offsets[e] + counts[e]; r < offsets[e + 1]; ++r) {",
                               "for (int64_t r = (int64_t)offsets[e] + counts[e]; r < offsets[e + 1] - 1; ++r) {"),
    "zero_padding_weights_kept": ("      if (expand_weights) expand_weights[r] = 0.0f;\n", ""),
    "compact_wrong_token": ("memcpy(recv_x + (int64_t)i * row_bytes, x + (int64_t)t * row_bytes, (size_t)row_bytes);",
                            "memcpy(recv_x + (int64_t)i * row_bytes, x + (int64_t)i * row_bytes, (size_t)row_bytes);"),
    "compact_mask_kept": ("recv_topk_idx[(int64_t)i * K + k] = dst_slot[tk] >= 0 ? topk_idx[tk] : -1;",
                          "recv_topk_idx[(int64_t)i * K + k] = topk_idx[tk];"),
    "compact_combine_unreceived_kept": ("    int32_t i = any ? row_of[t] : -1;", "    int32_t i = row_of[t] >= 0 ? row_of[t] : 0;"),
    "compact_combine_bias_dropped": ("        acc = acc + bf16_bits_to_float(bias[(int64_t)t * H + h]);\n", ""),
    "combine_reverse_k": ("      for (int32_t k = 0; k < K; ++k) {\n        if (d[k] < 0) continue;\n        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;\n        float v",
                          "      for (int32_t k = K - 1; k >= 0; --k) {\n        if (d[k] < 0) continue;\n        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;\n        float v"),
    "combine_f32_reverse_k": ("      for (int32_t k = 0; k < K; ++k) {\n        if (d[k] < 0) continue;\n        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;\n        float prod",
                              "      for (int32_t k = K - 1; k >= 0; --k) {\n        if (d[k] < 0) continue;\n        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;\n        float prod"),
    "combine_fma": ("        float prod = w * v;\n        acc = acc + prod;", "        acc = __builtin_fmaf(w, v, acc);"),
    "combine_f32_fma": ("        float prod = w * y[(int64_t)d[k] * H + h];\n        acc = acc + prod;",
                        "        acc = __builtin_fmaf(w, y[(int64_t)d[k] * H + h], acc);"),
    "compact_f32_bias_dropped": ("      if (bias) v = v + bias[(int64_t)t * H + h];\n", ""),
    "compact_f32_unreceived_kept": ("const float *row = received && recv_row[t] >= 0 ? y + (int64_t)recv_row[t] * H : NULL;",
                                    "const float *row = y + (int64_t)(recv_row[t] >= 0 ? recv_row[t] : 0) * H;"),
    "compact_f32_bias_first": ("      float v = row ? row[h] : 0.0f;\n      if (bias) v = v + bias[(int64_t)t * H + h];",
                               "      float v = bias ? bias[(int64_t)t * H + h] : 0.0f;\n      if (row) v = v + row[h];"),
    "compact_f32_row_zero": ("float v = row ? row[h] : 0.0f;", "float v = row ? row[0] : 0.0f;"),
    "combine_f32_weight_k0": ("        float w = topk_weights ? topk_weights[(int64_t)t * K + k] : 1.0f;\n        float prod",
                              "        float w = topk_weights ? topk_weights[(int64_t)t * K] : 1.0f;\n        float prod"),
}


def _run_pins(libpath):
    """Run the pin suite against the oracle at libpath; return the list of pins that failed."""
    failed = []

    def attempt(name, fn):
        try:
            fn()
        except (AssertionError, ValueError) as exc:  # noqa: F841
            failed.append(name)

    import json
    g = os.path.join(os.path.dirname(__file__), "golden")
    lay_gold = json.load(open(os.path.join(g, "layout_worked_examples.json")))
    comb_gold = json.load(open(os.path.join(g, "combine_worked_examples.json")))

    def golden_layout():
        for c in lay_gold["cases"]:
            res = oracle.layout(np.array(c["topk_idx"], np.int32), c["E"], c["A"], _lib=libpath)
            pins.check_layout_matches(res, np.array(c["counts"]), np.array(c["offsets"]),
                                      np.array(c["dst_slot"]), np.array(c["recv_src_metadata"]))

    def golden_combine():
        h = lambda v: int(v, 16)  # noqa: E731
        for r in comb_gold["rounding"]:
            f = np.array([h(r["f32_hex"])], np.uint32).view(np.float32)[0]
            assert oracle.f32_to_bf16(f, _lib=libpath) == h(r["bf16_hex"])
        for nan_bits in (0x7FFFFFFF, 0xFFFFFFFF):
            b = oracle.f32_to_bf16(np.array([nan_bits], np.uint32).view(np.float32)[0], _lib=libpath)
            assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0
        for c in comb_gold["combine"]:
            y = np.array([[h(v) for v in row] for row in c["y_rows_hex"]], np.uint16)
            w = None if c["topk_weights"] is None else np.array(c["topk_weights"], np.float32)
            out = oracle.combine(y, np.array(c["dst_slot"], np.int32), w, _lib=libpath)
            assert np.array_equal(out, np.array([[h(v) for v in r] for r in c["out_hex"]], np.uint16))

    def bruteforce_and_invariants():
        for seed, (T, E, K, A) in enumerate([(7, 4, 3, 2), (9, 5, 2, 3), (12, 8, 4, 4)]):
            g_ = np.random.default_rng([seed, 7])
            idx = I.routing_uniform(g_, T, E, K)
            idx[g_.random(idx.shape) < 0.2] = -1
            res = oracle.layout(idx, E, A, _lib=libpath)
            c, o, d, rows = pins.layout_bruteforce(idx, E, A)
            pins.check_layout_matches(res, c, o, d, np.array(rows, np.int64).reshape(-1, K + 2))
            pins.check_layout_invariants(idx, E, A, res)

    def argsort_mid():
        idx = I.routing_uniform(np.random.default_rng(3), 300, 64, 8)
        res = oracle.layout(idx, 64, 16, _lib=libpath)
        pins.check_layout_matches(res, *pins.layout_by_argsort(idx, 64, 16))

    w = I.custom("mut", 77, 40, 256, 16, 4, 2)
    case = I.make_case(w)
    ref_lay = pins.layout_by_argsort(case.topk_idx, w.E, w.A)
    dst = ref_lay[2].astype(np.int32)

    def dispatch_pins():
        before = np.full((w.cap, w.H * 2), 0x5A, np.uint8)
        X, _, Xw = oracle.dispatch(case.x, dst, w.cap, topk_weights=case.topk_weights,
                                   expand_x=before.copy(), _lib=libpath)
        pins.check_dispatch(case.x.view(np.uint8).reshape(w.T, -1), dst, before, X)
        assert np.array_equal(Xw[dst.ravel()], case.topk_weights.ravel())
        wf = I.custom("mutf8", 78, 30, 256, 8, 2, 1, I.FP8_E4M3)
        cf = I.make_case(wf, with_y=False)
        df = pins.layout_by_argsort(cf.topk_idx, wf.E, wf.A)[2].astype(np.int32)
        bs = np.zeros((wf.cap, 2), np.float32)
        _, Xs, _ = oracle.dispatch(cf.x, df, wf.cap, x_scales=cf.x_scales, expand_scales=bs.copy(),
                                   _lib=libpath)
        pins.check_dispatch(cf.x_scales.view(np.uint8).reshape(wf.T, -1), df,
                            bs.view(np.uint8).reshape(wf.cap, -1), Xs.view(np.uint8).reshape(wf.cap, -1))

    def combine_bound():
        for wts in (case.topk_weights, None):
            out = oracle.combine(case.y, dst, wts, _lib=libpath)
            pins.check_combine_bound(case.y, dst, wts, out)

    def identity():
        X, _, _ = oracle.dispatch(case.x, dst, w.cap, _lib=libpath)
        out = oracle.combine(X.view(np.uint16).reshape(w.cap, w.H), dst, case.topk_weights, _lib=libpath)
        assert np.array_equal(out, case.x)

    def bias_pins():
        h = lambda v: int(v, 16)  # noqa: E731
        for c in comb_gold["combine_bias"]:
            y = np.array([[h(v) for v in row] for row in c["y_rows_hex"]], np.uint16)
            b = np.array([[h(v) for v in row] for row in c["bias_hex"]], np.uint16)
            out = oracle.combine(y, np.array(c["dst_slot"], np.int32), None, b, _lib=libpath)
            assert np.array_equal(out, np.array([[h(v) for v in r] for r in c["out_hex"]], np.uint16))
        for c in comb_gold["combine_f32_bias"]:
            out = oracle.combine_f32(np.array(c["y_rows"], np.float32), np.array(c["dst_slot"], np.int32),
                                     np.array(c["topk_weights"], np.float32),
                                     np.array(c["bias"], np.float32), _lib=libpath)
            assert np.array_equal(out.view(np.uint32), np.array(c["out"], np.float32).view(np.uint32))
        bias = np.random.default_rng(8).integers(0, 0x3f00, (w.T, w.H)).astype(np.uint16)
        pins.check_combine_bound(case.y, dst, case.topk_weights,
                                 oracle.combine(case.y, dst, case.topk_weights, bias, _lib=libpath), bias)

    def zero_padding_pins():
        wz = I.custom("mutzp", 79, 120, 256, 16, 4, 8)
        idx = I.make_routing(wz.routing, wz.seed, wz.T, wz.E, wz.K)
        counts, offsets, _, _ = pins.layout_by_argsort(idx, wz.E, wz.A)
        g = np.random.default_rng(1)
        X = g.integers(1, 256, (wz.cap, wz.H), dtype=np.uint8)
        Wt = g.random(wz.cap).astype(np.float32) + 1
        before = (X.copy(), Wt.copy())
        oracle.zero_padding(X, counts, offsets, None, Wt, _lib=libpath)
        pad = np.zeros(wz.cap, bool)
        for e in range(wz.E):
            pad[offsets[e] + counts[e]:offsets[e + 1]] = True
        for a, b in zip((X, Wt), before):
            assert np.all(a[pad] == 0) and np.array_equal(a[~pad], b[~pad])

    def non_expand_pins():
        h = lambda rows: np.array([[int(v, 16) for v in r] for r in rows], np.uint16)  # noqa: E731
        for c in lay_gold["non_expand"]:
            idx = np.array(c["topk_idx"], np.int32)
            dst_, meta_ = np.array(c["dst_slot"], np.int32), np.array(c["recv_src_metadata"], np.int32)
            rx, _, ri, _ = oracle.dispatch_compact(h(c["x_hex"]), idx, dst_, meta_, c["num_recv"], _lib=libpath)
            assert np.array_equal(rx.view(np.uint16), h(c["recv_x_hex"]))
            assert np.array_equal(ri, c["recv_topk_idx"])
            out = oracle.combine_compact(h(c["y_hex"]), dst_, meta_, c["num_recv"], h(c["bias_hex"]), _lib=libpath)
            assert np.array_equal(out, h(c["out_bias_hex"]))
            out = oracle.combine_compact(h(c["y_hex"]), dst_, meta_, c["num_recv"], _lib=libpath)
            assert np.array_equal(out, h(c["out_no_bias_hex"]))
            f = lambda rows: np.array(rows, np.float32)  # noqa: E731
            out = oracle.combine_compact_f32(f(c["y_f32"]), dst_, meta_, c["num_recv"], f(c["bias_f32"]),
                                             _lib=libpath)
            assert np.array_equal(out.view(np.uint32), f(c["out_f32_bias"]).view(np.uint32))
            out = oracle.combine_compact_f32(f(c["y_f32"]), dst_, meta_, c["num_recv"], _lib=libpath)
            assert np.array_equal(out.view(np.uint32), f(c["out_f32_no_bias"]).view(np.uint32))

    def combine_f32_pins():
        for c in comb_gold["combine_f32"]:
            out = oracle.combine_f32(np.array(c["y_rows"], np.float32), np.array(c["dst_slot"], np.int32),
                                     np.array(c["topk_weights"], np.float32), _lib=libpath)
            assert np.array_equal(out.view(np.uint32), np.array(c["out"], np.float32).view(np.uint32))
        yf = np.random.default_rng(5).standard_normal((w.cap, w.H)).astype(np.float32)
        for wts in (case.topk_weights, None):
            pins.check_combine_bound_f32(yf, dst, wts, oracle.combine_f32(yf, dst, wts, _lib=libpath))

    for name, fn in [("golden_layout", golden_layout), ("golden_combine", golden_combine),
                     ("combine_f32", combine_f32_pins), ("bias", bias_pins),
                     ("zero_padding", zero_padding_pins), ("non_expand", non_expand_pins),
                     ("bruteforce", bruteforce_and_invariants), ("argsort", argsort_mid),
                     ("dispatch", dispatch_pins), ("combine_bound", combine_bound),
                     ("identity", identity)]:
        attempt(name, fn)
    return failed


def _build_variant(tmp_path, name, find, repl, nth=None):
    src = open(obuild.SRC).read()
    if nth is None:
        assert src.count(find) == 1, f"mutation {name}: pattern must occur exactly once"
        at = src.index(find)
    else:  # the nth occurrence (0-based) of a pattern shared by several functions
        assert src.count(find) > nth, f"mutation {name}: pattern must occur at least {nth + 1} times"
        at = -1
        for _ in range(nth + 1):
            at = src.index(find, at + 1)
    p = tmp_path / f"{name}.c"
    p.write_text(src[:at] + repl + src[at + len(find):])
    out = str(tmp_path / f"lib{name}.so")
    flags = [f for f in obuild.CFLAGS if f not in ("-Werror", "-Wextra")]
    subprocess.run(["gcc", *flags, "-o", out, str(p)], check=True)
    return out


def test_unmutated_oracle_passes_every_pin():
    assert _run_pins(obuild.LIB) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    lib = _build_variant(tmp_path, name, *MUTANTS[name])
    failed = _run_pins(lib)
    assert failed, f"planted mistake {name!r} passed every pin"
