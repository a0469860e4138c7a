"""Seeded random sweep of shapes on the GPU against the CPU oracle.

Each case draws a compiled (hidden, topk, dtype), a token count, an expert
count up to 1024, an alignment, a masking fraction, out-of-range ids, an
optional bias and an optional workgroup cap, then runs layout, dispatch,
combine (and, for bf16, the non-expand pair, its combine also on binary32
rows) through the C ABI; even seeds also ask the layout for the dispatch plan
and dispatch through it, and seeds that are multiples of 3 hand the layout x
as its read-ahead region. A second
sweep draws batches that fit one layout tile and runs ep_layout_dispatch (one
launch), with or without router weights and scale rows. A third draws large
layouts alone (up to 70K tokens, every launch path of the layout). Bar as in
the other parity tests: everything bit-exact except bf16 combine (<= 1 ulp).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - only on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from combine_ep_layout_amd import binding as B  # noqa: E402
from combine_ep_layout_amd import inputs as I  # noqa: E402
from tests import pins  # noqa: E402
from tests.gpu_util import DEV, DeviceCase, dev_layout, layout_to_host, to_dev, to_host  # noqa: E402

HIDDEN = {I.BF16: [256, 512, 1024, 2048, 4096, 7168], I.FP32: [256, 512, 1024, 2048],
          I.FP8_E4M3: [512, 1024, 2048, 7168], I.FP4X2: [256, 512, 1024, 3584]}
TOPK = [1, 2, 4, 6, 8]


def draw(seed):
    g = np.random.default_rng([seed, 4242])
    dtype = int(g.choice([I.BF16, I.BF16, I.FP32, I.FP8_E4M3, I.FP4X2]))
    H = int(g.choice(HIDDEN[dtype]))
    K = int(g.choice(TOPK))
    E = int(g.choice([K, 16, 64, 256, 512, 1024]))
    E = max(E, K)
    T = int(g.integers(1, 2500 if H <= 2048 else 1200))
    A = int(g.choice([1, 2, 16, 128]))
    mask = float(g.choice([0.0, 0.0, 0.1, 0.5]))
    bias = bool(g.integers(0, 2))
    cap = int(g.choice([0, 0, 0, 3, 40]))
    scales = bool(g.integers(0, 2))
    return dict(dtype=dtype, H=H, K=K, E=E, T=T, A=A, mask=mask, bias=bias, cap=cap, scales=scales)


@pytest.mark.parametrize("seed", range(48))
def test_random_shape(seed):
    c = draw(seed)
    print(f"random case {seed}: {c}", flush=True)
    out_dtype = I.FP32 if c["dtype"] == I.FP32 else I.BF16
    w = I.custom(f"rnd{seed}", 3000 + seed, c["T"], c["H"], c["E"], c["K"], c["A"], c["dtype"],
                 "uniform", out_dtype=out_dtype, scales=c["scales"])
    case = I.make_case(w, mask_frac=c["mask"])
    case.topk_idx[::11, 0] = w.E + 1  # some ids outside [0, E): masked
    plan = seed % 2 == 0
    s = torch.cuda.Stream()
    try:
        B.ep_set_workgroup_limit(s, c["cap"])
        with torch.cuda.stream(s):
            dc = DeviceCase(case)
            lay = dc.layout(stream=s, plan=plan, read_ahead=seed % 3 == 0)
            dc.dispatch(stream=s, plan=plan)
            bias = None
            if c["bias"]:
                bias_host = (I.normal_f32(w.seed, 9, w.T, dc.H_out) if out_dtype == I.FP32
                             else I.normal_bf16(w.seed, 9, w.T, dc.H_out))
                bias = to_dev(bias_host)
            out = dc.combine(bias=bias, stream=s)
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)

    ref = oracle.layout(case.topk_idx, w.E, w.A)
    got = layout_to_host(lay)
    for k in ("counts", "offsets", "dst_slot"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["num_recv"] == ref["num_recv"]
    assert np.array_equal(got["recv_src_metadata"], ref["recv_src_metadata"])
    if plan:
        assert np.array_equal(to_host(lay["plan"]), pins.dispatch_plan(ref["dst_slot"], w.E, w.K))

    X = np.full((w.cap, dc.row_bytes), dc.sentinel, np.uint8)
    Xs = (np.full((w.cap, case.x_scales.shape[1]), -3.0, np.float32)
          if case.x_scales is not None else None)
    Xw = np.full(w.cap, -5.0, np.float32)
    oracle.dispatch(case.x, ref["dst_slot"], w.cap, x_scales=case.x_scales,
                    topk_weights=case.topk_weights, expand_x=X, expand_scales=Xs, expand_weights=Xw)
    assert np.array_equal(to_host(dc.expand_x), X), "expand_x"
    assert np.array_equal(to_host(dc.expand_w).view(np.uint32), Xw.view(np.uint32)), "weights"
    if Xs is not None:
        assert np.array_equal(to_host(dc.expand_s).view(np.uint32), Xs.view(np.uint32)), "scales"

    bias_h = None if bias is None else bias_host
    if out_dtype == I.FP32:
        want = oracle.combine_f32(case.y, ref["dst_slot"], case.topk_weights, bias_h)
        assert np.array_equal(to_host(out).view(np.uint32), want.view(np.uint32)), "combine"
    else:
        want = oracle.combine(case.y, ref["dst_slot"], case.topk_weights, bias_h)
        d = pins.bf16_ulp_distance(to_host(out, np.uint16), want)
        print(f"  combine exact={np.mean(d == 0):.6f} max_ulp={int(d.max())}", flush=True)
        assert d.max() <= 1

    if c["dtype"] == I.BF16:  # the non-expand pair on the same layout
        n = ref["num_recv"]
        recv_x = torch.full((w.T, dc.row_bytes), 0x5A, dtype=torch.uint8, device=DEV)
        recv_i = torch.full((w.T, w.K), -7, dtype=torch.int32, device=DEV)
        B.ep_dispatch_compact(dc.x, None, dc.idx, None, lay["dst_slot"], lay["meta"],
                              lay["num_recv"], w.T, w.H, w.K, w.dtype, recv_x, None, recv_i, None)
        out2 = torch.empty((w.T, w.H), dtype=torch.int16, device=DEV)
        B.ep_combine_compact(dc.y, bias, lay["dst_slot"], lay["meta"], lay["num_recv"], w.T, w.H,
                             w.K, B.EP_BF16, out2)
        torch.cuda.synchronize()
        rx, _, ri, _ = oracle.dispatch_compact(case.x, case.topk_idx, ref["dst_slot"],
                                               ref["recv_src_metadata"], n)
        assert np.array_equal(to_host(recv_x)[:n], rx) and np.array_equal(to_host(recv_i)[:n], ri)
        want2 = oracle.combine_compact(case.y[:max(n, 1)], ref["dst_slot"], ref["recv_src_metadata"],
                                       n, bias_h)
        assert pins.bf16_ulp_distance(to_host(out2, np.uint16), want2).max() <= 1
        # binary32 rows through the same non-expand combine
        y32 = I.normal_f32(w.seed, 4, max(w.T, 1), w.H)
        b32 = I.normal_f32(w.seed, 9, w.T, w.H) if c["bias"] else None
        out3 = torch.empty((w.T, w.H), dtype=torch.float32, device=DEV)
        y32_d, b32_d = to_dev(y32), (to_dev(b32) if b32 is not None else None)
        torch.cuda.synchronize()
        B.ep_combine_compact(y32_d, b32_d, lay["dst_slot"], lay["meta"], lay["num_recv"], w.T, w.H,
                             w.K, B.EP_FP32, out3)
        torch.cuda.synchronize()
        want3 = oracle.combine_compact_f32(y32, ref["dst_slot"], ref["recv_src_metadata"], n, b32)
        assert np.array_equal(to_host(out3).view(np.uint32), want3.view(np.uint32)), "fp32 compact"


def draw_one_tile(seed):
    g = np.random.default_rng([seed, 777])
    dtype = int(g.choice([I.BF16, I.BF16, I.FP32, I.FP8_E4M3, I.FP4X2]))
    H = int(g.choice(HIDDEN[dtype]))
    K = int(g.choice(TOPK))
    E = max(K, int(g.choice([K, 16, 64, 256, 300, 1024])))
    entries = 1024 if E <= 256 else (512 if E <= 512 else 256)  # one layout tile
    T = int(g.integers(1, entries // K + 1))
    A = int(g.choice([1, 2, 16, 128]))
    mask = float(g.choice([0.0, 0.1, 0.5])) if T > 1 else 0.0
    scales = bool(g.integers(0, 2)) and dtype in (I.FP8_E4M3, I.FP4X2)
    weights = bool(g.integers(0, 2))
    cap = int(g.choice([0, 0, 0, 1, 5, 64]))
    return dict(dtype=dtype, H=H, K=K, E=E, T=T, A=A, mask=mask, scales=scales, weights=weights,
                cap=cap)


@pytest.mark.parametrize("seed", range(40))
def test_random_one_tile_layout_dispatch(seed):
    c = draw_one_tile(seed)
    print(f"one-tile case {seed}: {c}", flush=True)
    w = I.custom(f"rndf{seed}", 7000 + seed, c["T"], c["H"], c["E"], c["K"], c["A"], c["dtype"],
                 "uniform", scales=c["scales"])
    case = I.make_case(w, with_y=False, mask_frac=c["mask"])
    case.topk_idx[::11, 0] = w.E + 1  # some ids outside [0, E): masked
    dc = DeviceCase(case, with_y=False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # the inputs and buffers were written there
    try:
        B.ep_set_workgroup_limit(s, c["cap"])
        with torch.cuda.stream(s):
            dc.layout_dispatch(stream=s, weights=c["weights"])
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)

    ref = oracle.layout(case.topk_idx, w.E, w.A)
    got = layout_to_host(dc.lay)
    for k in ("counts", "offsets", "dst_slot"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["num_recv"] == ref["num_recv"]
    assert np.array_equal(got["recv_src_metadata"], ref["recv_src_metadata"])

    X = np.full((w.cap, dc.row_bytes), dc.sentinel, np.uint8)
    Xs = (np.full((w.cap, case.x_scales.shape[1]), -3.0, np.float32)
          if case.x_scales is not None else None)
    Xw = np.full(w.cap, -5.0, np.float32)
    oracle.dispatch(case.x, ref["dst_slot"], w.cap, x_scales=case.x_scales,
                    topk_weights=case.topk_weights if c["weights"] else None, expand_x=X,
                    expand_scales=Xs, expand_weights=Xw)
    assert np.array_equal(to_host(dc.expand_x), X), "expand_x"
    assert np.array_equal(to_host(dc.expand_w).view(np.uint32), Xw.view(np.uint32)), "weights"
    if Xs is not None:
        assert np.array_equal(to_host(dc.expand_s).view(np.uint32), Xs.view(np.uint32)), "scales"


@pytest.mark.parametrize("seed", range(16))
def test_random_large_layout(seed):
    g = np.random.default_rng([seed, 31337])
    K = int(g.choice(TOPK))
    E = max(K, int(g.choice([8, 64, 256, 300, 512, 777, 1024])))
    T = int(g.choice([int(g.integers(1, 3000)), int(g.integers(3000, 70000))]))
    A = int(g.choice([1, 4, 128]))
    mask = float(g.choice([0.0, 0.05, 0.5]))
    cap = int(g.choice([0, 0, 0, 1, 7, 33, 200]))
    plan = bool(g.integers(0, 2))
    print(f"large layout {seed}: T={T} K={K} E={E} A={A} mask={mask} cap={cap} plan={plan}",
          flush=True)
    if T * E <= 10_000_000:  # distinct experts per token
        idx = np.argsort(g.random((T, E)), axis=1)[:, :K].astype(np.int32)
    else:  # repeats allowed: each entry still gets its own row
        idx = g.integers(0, E, (T, K)).astype(np.int32)
    idx[g.random((T, K)) < mask] = -1
    idx[::13, 0] = E + 3  # outside [0, E): masked
    ref = oracle.layout(idx, E, A)
    s = torch.cuda.Stream()
    try:
        B.ep_set_workgroup_limit(s, cap)
        with torch.cuda.stream(s):
            lay = dev_layout(to_dev(idx), T, K, E, A, T * K + E * (A - 1), plan=plan, stream=s)
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)
    got = layout_to_host(lay)
    for k in ("counts", "offsets", "dst_slot"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["num_recv"] == ref["num_recv"]
    assert np.array_equal(got["recv_src_metadata"], ref["recv_src_metadata"])
    if plan:
        assert np.array_equal(to_host(lay["plan"]), pins.dispatch_plan(ref["dst_slot"], E, K))
