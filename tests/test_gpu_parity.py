"""GPU path vs the CPU oracle, through the C ABI (needs an MI355X).

Bar: layout, metadata and dispatch bytes bit-exact; combine within 1 bf16
ulp (ordered bit-pattern distance <= 1; the kernels use the same binary32
operation order as the oracle, so the tests also report exact matches).
Covers the five workloads at full size (in the launch configuration the
benchmark times), small shapes spanning several layout tiles with ragged
tails, masking, empty and degenerate inputs, and special values.
"""
import json
import os

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
from tests.gpu_util import DeviceCase, dev_layout, layout_to_host, to_dev, to_host  # noqa: E402
import bench  # noqa: E402  (the launch configuration it times)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(msg):
    print(msg, flush=True)


def check_layout(got, ref):
    assert np.array_equal(got["counts"], ref["counts"]), "counts"
    assert np.array_equal(got["offsets"], ref["offsets"]), "offsets"
    assert np.array_equal(got["dst_slot"], ref["dst_slot"]), "dst_slot"
    assert got["num_recv"] == ref["num_recv"], "num_recv"
    assert np.array_equal(got["recv_src_metadata"], ref["recv_src_metadata"]), "recv_src_metadata"
    # rows past num_recv are not written
    assert np.all(got["meta_full"][ref["num_recv"]:] == -7)


def check_dispatch(dc: DeviceCase, ref_dst):
    w, case = dc.w, dc.case
    got = to_host(dc.expand_x)
    xb = case.x.view(np.uint8).reshape(w.T, -1)
    before = np.full_like(got, dc.sentinel)
    pins.check_dispatch(xb, ref_dst, before, got)
    v = ref_dst >= 0
    gw = to_host(dc.expand_w)
    assert np.array_equal(gw[ref_dst[v]], case.topk_weights[v]), "expand_weights"
    untouched = np.ones(w.cap, bool)
    untouched[ref_dst[v]] = False
    assert np.all(gw[untouched] == -5.0), "padding weights untouched"
    if dc.expand_s is not None:
        gs = to_host(dc.expand_s)
        pins.check_dispatch(case.x_scales.view(np.uint8).reshape(w.T, -1), ref_dst,
                            np.full_like(gs, -3.0).view(np.uint8), gs.view(np.uint8))


def check_combine(got_bits, ref_bits, label=""):
    d = pins.bf16_ulp_distance(got_bits, ref_bits)
    exact = int((d == 0).sum())
    _say(f"combine {label}: {exact}/{d.size} exact, max ulp distance {int(d.max()) if d.size else 0}")
    assert d.size == 0 or d.max() <= 1, f"combine beyond 1 bf16 ulp: {int((d > 1).sum())} elements"


@pytest.mark.parametrize("config", ["bench", "separate"])
@pytest.mark.parametrize("name", list(I.WORKLOADS))
def test_workload_full_size(name, config):
    """Every workload at full size, in the launch configuration the benchmark times
    ("bench": ep_layout_dispatch for a batch of one layout tile, else the layout with
    the dispatch plan and the planned dispatch) and as separate plain calls."""
    w = I.WORKLOADS[name]
    fused = bench.one_layout_tile(w.T, w.K, w.E)
    _say(f"[workload {name}, {config}{' (one call)' if config == 'bench' and fused else ''}] "
         f"T={w.T} H={w.H} E={w.E} K={w.K} A={w.A} dtype={w.dtype} cap={w.cap}")
    case = I.make_case(w)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case)
    if config == "bench" and fused:
        dc.layout_dispatch()
    elif config == "bench":
        dc.layout(plan=True)
        dc.dispatch(plan=True)
    else:
        dc.layout()
        dc.dispatch()
    out = dc.combine()
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])
    ref_out = oracle.combine(case.y, ref["dst_slot"], case.topk_weights)
    check_combine(to_host(out, np.uint16), ref_out, name)


@pytest.mark.parametrize("name", ["prefill_fp4x2", "prefill_fp32_combine", "prefill_fp32"])
def test_dtype_variant_full_size(name):
    """The prefill shape with the other row types, at full size and in the launch
    configuration the benchmark times (layout with the dispatch plan, the plan
    walked): fp4x2 rows with scale rows, bf16 rows with fp32 combine rows, and
    fp32 throughout. Layout and dispatch bit-exact; combine 1 ulp (bf16 rows)
    or bit-exact (fp32 rows)."""
    w = I.EXTRA_WORKLOADS[name]
    _say(f"[workload {name}] T={w.T} H={w.H} E={w.E} K={w.K} A={w.A} dtype={w.dtype} "
         f"out_dtype={w.out_dtype} cap={w.cap}")
    case = I.make_case(w)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case)
    dc.layout(plan=True)
    dc.dispatch(plan=True)
    out = dc.combine()
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])
    if w.out_dtype == I.FP32:
        want = oracle.combine_f32(case.y, ref["dst_slot"], case.topk_weights)
        assert np.array_equal(to_host(out, np.float32).view(np.uint32), want.view(np.uint32)), \
            "fp32 combine not bit-exact"
    else:
        check_combine(to_host(out, np.uint16), oracle.combine(case.y, ref["dst_slot"],
                                                              case.topk_weights), name)
    del dc, out
    torch.cuda.empty_cache()


RAGGED = [
    # T, H, E, K, A, mask, dtype, routing
    (1000, 256, 16, 2, 1, 0.0, I.BF16, "uniform"),
    (1500, 512, 64, 8, 4, 0.0, I.BF16, "uniform"),
    (777, 1024, 256, 6, 16, 0.1, I.BF16, "uniform"),
    (300, 2048, 1024, 4, 1, 0.0, I.BF16, "uniform"),
    (3000, 256, 1, 1, 8, 0.0, I.BF16, "uniform"),
    (129, 7168, 256, 8, 128, 0.0, I.BF16, "uniform"),
    (128, 7168, 256, 8, 1, 0.0, I.BF16, "zipf"),
    (4097, 256, 256, 8, 128, 0.02, I.BF16, "uniform"),
    (513, 1024, 32, 4, 2, 0.0, I.FP8_E4M3, "hot8"),
    (200, 256, 8, 2, 1, 1.0, I.BF16, "uniform"),
    (1, 4096, 128, 8, 32, 0.0, I.BF16, "uniform"),
    (2049, 512, 300, 8, 7, 0.05, I.BF16, "zipf"),
    (40, 256, 1024, 6, 3, 0.1, I.BF16, "uniform"),      # one tile of 4 waves (E > 512)
    (64, 256, 512, 8, 2, 0.0, I.BF16, "zipf"),          # one tile of 8 waves (256 < E <= 512)
    (1100, 1024, 512, 2, 5, 0.0, I.FP8_E4M3, "uniform"),
    # above 2^14 entries: the two-launch layout path with a workspace
    (20000, 256, 256, 8, 4, 0.01, I.BF16, "uniform"),
    (70001, 256, 64, 2, 1, 0.0, I.BF16, "zipf"),
    (40000, 256, 1024, 4, 2, 0.0, I.BF16, "uniform"),
    (22000, 512, 300, 6, 3, 0.02, I.FP8_E4M3, "hot8"),
]


@pytest.mark.parametrize("T,H,E,K,A,mask,dtype,routing", RAGGED)
def test_ragged_shapes(T, H, E, K, A, mask, dtype, routing):
    w = I.custom(f"r{T}_{H}_{E}_{K}", 1000 + T, T, H, E, K, A, dtype, routing)
    _say(f"[ragged] {w}")
    case = I.make_case(w, mask_frac=mask)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case)
    dc.layout()
    dc.dispatch()
    out = dc.combine()
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])
    check_combine(to_host(out, np.uint16), oracle.combine(case.y, ref["dst_slot"], case.topk_weights),
                  w.name)
    # unweighted combine (weight 1)
    out = dc.combine(weights=False)
    check_combine(to_host(out, np.uint16), oracle.combine(case.y, ref["dst_slot"], None), "w=1")


# x larger than 128 MiB: the uncapped dispatch switches to one wave per source
# slice and group of entries (groups of 4 for K = 8 and 4, 3 for K = 6, 2 for
# K = 2); each case sits just past that size, with masking and ragged T.
BEYOND_CACHE = [
    # T, H, E, K, A, mask, dtype, scales
    (9500, 7168, 256, 8, 128, 0.02, I.BF16, False),
    (19001, 7168, 256, 6, 1, 0.05, I.FP8_E4M3, True),
    (16401, 2048, 64, 2, 4, 0.0, I.FP32, False),
    (37500, 3584, 128, 4, 1, 0.01, I.FP4X2, True),
]


@pytest.mark.parametrize("T,H,E,K,A,mask,dtype,scales", BEYOND_CACHE)
def test_dispatch_x_beyond_cache(T, H, E, K, A, mask, dtype, scales):
    w = I.custom(f"big{T}_{H}_{K}", 5000 + T, T, H, E, K, A, dtype, "uniform", scales=scales)
    _say(f"[x beyond cache] {w}")
    case = I.make_case(w, with_y=False, mask_frac=mask)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    dc.layout()
    dc.dispatch()
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])
    # without router weights no weight slot is written
    dc.expand_w.fill_(-5.0)
    dc.dispatch(weights=False)
    torch.cuda.synchronize()
    assert bool((dc.expand_w == -5.0).all())


# Combine shapes on both sides of the switch between the row-streaming
# kernel (at least 1024 tokens; one wave per token, or per piece of at most 14
# chunks of 16 bytes per lane) and the sliced kernel: masking (some tokens
# lose every entry), bias, K = 1 and 6, fp32 rows.
ROW_STREAM = [
    # T, H, E, K, A, mask, dtype, out_dtype
    (1024, 7168, 256, 8, 128, 0.3, I.BF16, I.BF16),
    (1023, 7168, 256, 8, 128, 0.3, I.BF16, I.BF16),
    (1024, 2048, 64, 6, 1, 0.1, I.BF16, I.BF16),
    (3000, 4096, 128, 1, 4, 0.05, I.BF16, I.BF16),
    (1500, 1024, 32, 4, 2, 0.2, I.FP32, I.FP32),
    (2500, 2048, 256, 2, 1, 0.6, I.FP32, I.FP32),
    # fp32 rows wider than one wave's registers: two pieces per token
    (1100, 7168, 256, 8, 1, 0.1, I.BF16, I.FP32),
    (1024, 4096, 64, 4, 1, 0.2, I.FP32, I.FP32),
    (1000, 7168, 256, 6, 1, 0.1, I.BF16, I.FP32),
]


@pytest.mark.parametrize("T,H,E,K,A,mask,dtype,out_dtype", ROW_STREAM)
def test_combine_row_stream(T, H, E, K, A, mask, dtype, out_dtype):
    w = I.custom(f"rs{T}_{H}_{K}", 7000 + T + K, T, H, E, K, A, dtype, "uniform",
                 out_dtype=out_dtype)
    _say(f"[combine stream] {w}")
    case = I.make_case(w, mask_frac=mask)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case)
    dc.layout()
    if out_dtype == I.FP32:
        bias_h = I.normal_f32(w.seed, 9, w.T, dc.H_out)
    else:
        bias_h = I.normal_bf16(w.seed, 9, w.T, dc.H_out)
    for weights, bias in ((True, None), (True, bias_h), (False, bias_h)):
        out = dc.combine(weights=weights, bias=None if bias is None else to_dev(bias))
        torch.cuda.synchronize()
        wts = case.topk_weights if weights else None
        label = f"{w.name} weights={weights} bias={bias is not None}"
        if out_dtype == I.FP32:
            want = oracle.combine_f32(case.y, ref["dst_slot"], wts, bias)
            got = to_host(out)
            same = got.view(np.uint32) == want.view(np.uint32)
            _say(f"combine fp32 {label}: {int(same.sum())}/{same.size} bit-exact")
            assert same.all(), label
        else:
            check_combine(to_host(out, np.uint16),
                          oracle.combine(case.y, ref["dst_slot"], wts, bias), label)


# Slots outside [0, capacity_rows) given straight to dispatch and combine are
# skipped like masked entries: every dispatch kernel (per (token, k), grouped
# for x beyond 128 MiB, capped fan-out) and every combine kernel (row-
# streaming, sliced, capped).
OUTSIDE = [
    # T, H, K, workgroup cap, run combine
    (2000, 7168, 8, 0, True),
    (600, 7168, 6, 0, True),
    (9500, 7168, 8, 0, False),
    (2000, 2048, 8, 16, True),
]


@pytest.mark.parametrize("T,H,K,wg_cap,do_combine", OUTSIDE)
def test_slots_outside_capacity_are_skipped(T, H, K, wg_cap, do_combine):
    w = I.custom(f"oob{T}_{H}_{K}", 9100 + T, T, H, 256, K, 1, I.BF16, "uniform")
    _say(f"[slots outside capacity] {w} workgroup cap {wg_cap}")
    case = I.make_case(w, with_y=do_combine)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dst = ref["dst_slot"].copy()
    pick = np.random.default_rng(9100 + T).random(dst.shape)
    dst[pick < 0.05] = w.cap  # the first row past the buffer
    dst[(pick >= 0.05) & (pick < 0.08)] = np.iinfo(np.int32).max
    dst[(pick >= 0.08) & (pick < 0.10)] = -7
    eff = np.where((dst >= 0) & (dst < w.cap), dst, -1).astype(np.int32)  # the header's meaning
    dc = DeviceCase(case, with_y=do_combine)
    dc.lay = {"dst_slot": to_dev(dst)}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # the inputs and buffers were written there
    try:
        B.ep_set_workgroup_limit(s, wg_cap)
        with torch.cuda.stream(s):
            dc.dispatch(stream=s)
            out = dc.combine(stream=s) if do_combine else None
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)
    X = np.full((w.cap, dc.row_bytes), dc.sentinel, np.uint8)
    Xw = np.full(w.cap, -5.0, np.float32)
    oracle.dispatch(case.x, eff, w.cap, topk_weights=case.topk_weights, expand_x=X,
                    expand_weights=Xw)
    assert np.array_equal(to_host(dc.expand_x), X), "expand_x"
    assert np.array_equal(to_host(dc.expand_w).view(np.uint32), Xw.view(np.uint32)), "weights"
    if do_combine:
        check_combine(to_host(out, np.uint16), oracle.combine(case.y, eff, case.topk_weights),
                      w.name)


PLANS = [
    # T, H, E, K, A, mask, workgroup cap, dtype: every layout launch shape, capped loops
    (100, 7168, 256, 8, 128, 0.1, 0, I.BF16),     # one tile
    (1500, 2048, 256, 8, 4, 0.05, 0, I.BF16),     # single launch, several tiles
    (4096, 7168, 256, 8, 128, 0.0, 0, I.BF16),    # two launches (the prefill shape)
    (20000, 256, 1024, 8, 4, 0.05, 0, I.BF16),    # with the tile-scan launch, 32-token tiles
    (3000, 1024, 300, 6, 3, 0.1, 0, I.BF16),      # 85-token tiles
    (5000, 512, 16, 1, 1, 0.2, 0, I.BF16),        # K = 1
    (4096, 7168, 256, 8, 128, 0.02, 3, I.BF16),   # capped: tiles loop; dispatch ignores the plan
    (1500, 2048, 256, 8, 4, 0.05, 5, I.BF16),
    (2048, 7168, 256, 8, 1, 0.05, 0, I.FP8_E4M3),  # scale rows ride with the planned walk
    (1024, 3584, 64, 6, 16, 0.1, 0, I.FP4X2),
]


@pytest.mark.parametrize("T,H,E,K,A,mask,wg_cap,dtype", PLANS)
def test_dispatch_plan(T, H, E, K, A, mask, wg_cap, dtype):
    w = I.custom(f"plan{T}_{E}_{K}", 9300 + T + E, T, H, E, K, A, dtype, "uniform")
    _say(f"[dispatch plan] {w} workgroup cap {wg_cap}")
    case = I.make_case(w, with_y=False, mask_frac=mask)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # the inputs and buffers were written there
    try:
        B.ep_set_workgroup_limit(s, wg_cap)
        with torch.cuda.stream(s):
            dc.layout(stream=s, plan=True)
            dc.dispatch(stream=s, plan=True)
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)
    check_layout(layout_to_host(dc.lay), ref)  # the plan changes no other output
    got = to_host(dc.lay["plan"])
    want = pins.dispatch_plan(ref["dst_slot"], w.E, w.K)
    assert np.array_equal(got, want), f"plan differs at {int(np.argmax((got != want).any(1)))}"
    check_dispatch(dc, ref["dst_slot"])


READ_AHEAD = [
    # T, E, K, A, read-ahead bytes, workgroup cap: every layout launch shape
    (100, 256, 8, 1, 100 * 14336, 0),            # one tile
    (1024, 64, 8, 1, 1024 * 14336, 0),           # one launch over 8 tiles
    (4096, 256, 8, 128, 4096 * 14336, 0),        # two launches, split read-ahead
    (20000, 1024, 8, 4, 20000 * 512 + 1000, 0),  # tile scan; not whole 128-byte lines
    (4096, 256, 8, 128, 200 << 20, 0),           # beyond the 128 MiB it reads
    (4096, 256, 8, 128, 4096 * 14336, 7),        # capped: ignored
    (333, 16, 2, 1, 3, 0),                       # less than one line
]


@pytest.mark.parametrize("T,E,K,A,nbytes,wg_cap", READ_AHEAD)
def test_layout_read_ahead_changes_nothing(T, E, K, A, nbytes, wg_cap):
    """ep_layout with a read-ahead region writes exactly what it writes without one."""
    _say(f"[read-ahead] T={T} E={E} K={K} A={A} bytes={nbytes} cap={wg_cap}")
    g = np.random.default_rng([T, E, 77])
    idx = I.routing_uniform(g, T, E, K)
    idx[g.random(idx.shape) < 0.05] = -1
    region = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    s = torch.cuda.Stream()
    try:
        B.ep_set_workgroup_limit(s, wg_cap)
        idx_d = to_dev(idx)
        torch.cuda.synchronize()
        lay = dev_layout(idx_d, T, K, E, A, T * K + E * (A - 1), stream=s, plan=True,
                         prefetch=region)
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)
    ref = oracle.layout(idx, E, A)
    check_layout(layout_to_host(lay), ref)
    assert np.array_equal(to_host(lay["plan"]), pins.dispatch_plan(ref["dst_slot"], E, K))


FUSED = [
    # T, H, E, K, A, mask, dtype, scales, routing, workgroup cap: one tile fuses layout and
    # dispatch into one launch; larger batches fall back to two
    (128, 7168, 256, 8, 1, 0.0, I.BF16, False, "zipf", 0),       # the decode shape
    (64, 256, 16, 2, 1, 0.0, I.BF16, False, "uniform", 0),       # tiny
    (100, 7168, 256, 8, 128, 0.1, I.FP8_E4M3, True, "uniform", 0),
    (100, 3584, 128, 8, 4, 0.05, I.FP4X2, True, "uniform", 0),
    (50, 1024, 32, 4, 2, 0.2, I.FP32, False, "uniform", 0),
    (170, 2048, 64, 6, 4, 0.1, I.BF16, False, "uniform", 0),     # 1020 entries, K = 6
    (64, 512, 300, 8, 1, 0.0, I.BF16, False, "uniform", 0),      # 512-entry tile
    (32, 512, 1024, 8, 3, 0.1, I.BF16, False, "uniform", 0),     # 256-entry tile
    (128, 7168, 256, 8, 1, 0.1, I.BF16, False, "zipf", 3),       # capped
    (4096, 7168, 256, 8, 128, 0.02, I.BF16, False, "uniform", 0),  # 32K entries: two launches
    (300, 1024, 64, 8, 1, 0.0, I.BF16, False, "uniform", 0),     # 3 tiles: two launches
    (1024, 7168, 64, 8, 1, 0.0, I.BF16, False, "uniform", 0),    # the MORI default shape, 8 tiles
    (2048, 7168, 256, 8, 128, 0.1, I.FP8_E4M3, True, "uniform", 0),  # 16 tiles, scale rows
    (1000, 3584, 128, 8, 4, 0.05, I.FP4X2, True, "uniform", 0),
    (700, 1024, 32, 4, 2, 0.2, I.FP32, False, "uniform", 0),
    (2700, 512, 64, 6, 4, 0.1, I.BF16, False, "uniform", 0),     # 16,200 entries, K = 6
    (900, 512, 300, 8, 1, 0.3, I.BF16, False, "uniform", 0),     # 512-entry tiles
    (1500, 512, 1024, 8, 3, 0.1, I.BF16, False, "uniform", 0),   # 256-entry tiles: 47 tiles
    (1024, 7168, 64, 8, 1, 0.1, I.BF16, False, "uniform", 7),    # capped
    # expert_alignment 1, uncapped: the copy workgroups count keys instead of ranking
    (128, 7168, 256, 8, 1, 0.3, I.BF16, False, "zipf", 0),       # decode shape, masked entries
    (100, 7168, 256, 8, 1, 0.1, I.FP8_E4M3, True, "uniform", 0),  # scale rows
    (100, 3584, 128, 8, 1, 0.05, I.FP4X2, True, "uniform", 0),
    (170, 2048, 64, 6, 1, 0.2, I.BF16, False, "uniform", 0),     # 1020 entries, K = 6
    (50, 1024, 32, 4, 1, 0.5, I.FP32, False, "uniform", 0),
    (64, 512, 300, 8, 1, 0.2, I.BF16, False, "uniform", 0),      # 512-entry tile, masked
    (32, 512, 1024, 8, 1, 0.1, I.BF16, False, "uniform", 0),     # 256-entry tile
    (1, 7168, 16, 2, 1, 0.0, I.BF16, False, "uniform", 0),       # one token
    (3, 256, 16, 1, 1, 0.0, I.BF16, False, "uniform", 0),        # 3 units, K = 1
]


@pytest.mark.parametrize("T,H,E,K,A,mask,dtype,scales,routing,wg_cap", FUSED)
def test_layout_dispatch(T, H, E, K, A, mask, dtype, scales, routing, wg_cap):
    w = I.custom(f"fused{T}_{E}_{K}", 9500 + T + E, T, H, E, K, A, dtype, routing,
                 scales=scales)
    _say(f"[layout + dispatch] {w} workgroup cap {wg_cap}")
    case = I.make_case(w, with_y=False, mask_frac=mask)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # the inputs and buffers were written there
    try:
        B.ep_set_workgroup_limit(s, wg_cap)
        with torch.cuda.stream(s):
            dc.layout_dispatch(stream=s)
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])


@pytest.mark.parametrize("T,H,E,K,A,dtype,scales,wg_cap", [
    (4096, 7168, 256, 8, 128, I.BF16, False, 0),      # 470 MB of rows: walks the plan
    (5000, 7168, 256, 8, 1, I.FP8_E4M3, True, 0),     # 296 MB of fp8 rows and scale rows
    (4096, 7168, 256, 8, 128, I.BF16, False, 16),     # capped: the fan-out ignores the plan
    (1024, 7168, 64, 8, 1, I.BF16, False, 0),         # the MORI default shape
    (300, 1024, 300, 6, 4, I.FP32, False, 0),         # 512-entry tiles, fp32 rows
    (3000, 512, 1024, 2, 16, I.FP4X2, True, 0),       # 256-entry tiles, fp4x2 with scale rows
])
def test_layout_dispatch_with_plan_workspace(T, H, E, K, A, dtype, scales, wg_cap):
    """ep_layout_dispatch given ep_layout_dispatch_workspace_bytes: several-tile batches
    walk a dispatch plan kept in the workspace; every output equals the oracle's."""
    w = I.custom(f"fused_pl{T}_{dtype}", 9700 + T, T, H, E, K, A, dtype, "uniform", scales=scales)
    _say(f"[layout + dispatch, plan workspace] {w} cap {wg_cap}")
    case = I.make_case(w, with_y=False, mask_frac=0.05)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    try:
        B.ep_set_workgroup_limit(s, wg_cap)
        with torch.cuda.stream(s):
            dc.layout_dispatch(stream=s, plan_workspace=True)
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])


@pytest.mark.parametrize("T,H,E,K,dtype,scales", [
    (128, 7168, 256, 8, I.BF16, False),     # the decode shape
    (100, 7168, 256, 8, I.FP8_E4M3, True),  # scale rows travel, weights do not
    (3, 512, 16, 1, I.BF16, False),         # 3 units for thousands of waves
    (1, 7168, 64, 8, I.BF16, False),        # one token
    (1024, 7168, 64, 8, I.BF16, False),     # 8 tiles: two launches
    (2048, 7168, 256, 8, I.FP8_E4M3, True),  # 16 tiles, scale rows
])
def test_layout_dispatch_without_weights(T, H, E, K, dtype, scales):
    """Without router weights to forward the expand weights stay untouched."""
    w = I.custom(f"fused_nw{T}_{K}", 9600 + T + K, T, H, E, K, 1, dtype, "uniform", scales=scales)
    _say(f"[layout + dispatch, no weights] {w}")
    case = I.make_case(w, with_y=False, mask_frac=0.1 if T > 1 else 0.0)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    dc.layout_dispatch(weights=False)
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    got = to_host(dc.expand_x)
    xb = case.x.view(np.uint8).reshape(w.T, -1)
    pins.check_dispatch(xb, ref["dst_slot"], np.full_like(got, dc.sentinel), got)
    assert np.all(to_host(dc.expand_w) == -5.0), "expand_weights untouched"
    if dc.expand_s is not None:
        gs = to_host(dc.expand_s)
        pins.check_dispatch(case.x_scales.view(np.uint8).reshape(w.T, -1), ref["dst_slot"],
                            np.full_like(gs, -3.0).view(np.uint8), gs.view(np.uint8))


def test_layout_dispatch_empty():
    w = I.custom("fused_empty", 9499, 0, 7168, 256, 8, 1)
    case = I.make_case(w, with_y=False)
    dc = DeviceCase(case, with_y=False)
    dc.layout_dispatch()
    torch.cuda.synchronize()
    got = layout_to_host(dc.lay)
    assert np.all(got["counts"] == 0) and np.all(got["offsets"] == 0) and got["num_recv"] == 0
    assert np.all(to_host(dc.expand_x) == dc.sentinel)


def test_empty_input():
    w = I.custom("empty", 5, 0, 256, 16, 2, 4)
    lay = dev_layout(None, 0, 2, 16, 4, w.cap)
    torch.cuda.synchronize()
    h = layout_to_host(lay)
    assert np.all(h["counts"] == 0) and np.all(h["offsets"] == 0) and h["num_recv"] == 0
    B.ep_dispatch(None, None, None, None, 0, 256, 2, B.EP_BF16, 0, None, None, None)
    B.ep_combine(None, None, None, None, 0, 256, 2, B.EP_BF16, 0, None)


def test_out_of_range_and_duplicate_ids():
    T, H, E, K, A = 300, 256, 12, 4, 3
    g = np.random.default_rng(9)
    idx = g.integers(-3, E + 4, (T, K)).astype(np.int32)  # duplicates, negatives, >= E
    w = I.custom("odd", 77, T, H, E, K, A)
    case = I.make_case(w)
    case.topk_idx = idx
    ref = oracle.layout(idx, E, A)
    dc = DeviceCase(case)
    dc.layout()
    dc.dispatch()
    out = dc.combine()
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])
    check_combine(to_host(out, np.uint16), oracle.combine(case.y, ref["dst_slot"], case.topk_weights))


@pytest.mark.parametrize("A", [1, 3])
def test_layout_dispatch_out_of_range_and_duplicate_ids(A):
    """The one-launch layout + dispatch with negative, out-of-range and repeated expert
    ids in one tile (alignment 1: the copy workgroups count keys; 3: they rank)."""
    T, H, E, K = 200, 256, 12, 4
    idx = np.random.default_rng(19).integers(-3, E + 4, (T, K)).astype(np.int32)
    w = I.custom(f"odd_fused{A}", 78, T, H, E, K, A)
    case = I.make_case(w, with_y=False)
    case.topk_idx = idx
    ref = oracle.layout(idx, E, A)
    dc = DeviceCase(case, with_y=False)
    dc.layout_dispatch()
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])


def test_identity_expert_round_trip_full_size():
    """dispatch -> identity expert (y = expand buffer) -> combine returns x bit-exactly."""
    w = I.WORKLOADS["prefill_aligned"]
    case = I.make_case(w, with_y=False)
    dc = DeviceCase(case, with_y=False)
    dc.layout()
    dc.dispatch()
    out = dc.combine(y=dc.expand_x)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out, np.uint16), case.x)


def test_repeat_runs_are_bit_identical():
    w = I.WORKLOADS["mori_default"]
    case = I.make_case(w)
    dc = DeviceCase(case)
    results = []
    for _ in range(2):
        dc.layout()
        dc.dispatch()
        out = dc.combine()
        torch.cuda.synchronize()
        results.append([to_host(dc.lay["dst_slot"]), to_host(dc.lay["meta"]), to_host(dc.expand_x),
                        to_host(out).copy()])
    for a, b in zip(*results):
        assert np.array_equal(a, b)


def test_combine_hand_worked_on_gpu():
    data = json.load(open(os.path.join(GOLDEN, "combine_worked_examples.json")))
    H = 256
    for c in data["combine"]:
        rows = np.zeros((len(c["y_rows_hex"]), H), np.uint16)
        for r, row in enumerate(c["y_rows_hex"]):
            rows[r, :len(row)] = [int(v, 16) for v in row]
        dst = np.array(c["dst_slot"], np.int32)
        wts_h = None if c["topk_weights"] is None else np.array(c["topk_weights"], np.float32)
        while not B.ep_supported(2, H, dst.shape[1], B.EP_BF16):  # pad with masked entries
            dst = np.concatenate([dst, np.full((dst.shape[0], 1), -1, np.int32)], axis=1)
            if wts_h is not None:
                wts_h = np.concatenate([wts_h, np.zeros((dst.shape[0], 1), np.float32)], axis=1)
        T, K = dst.shape
        wts = None if wts_h is None else to_dev(wts_h)
        out = torch.full((T, H), 0x7FC1, dtype=torch.int16, device="cuda:0")
        B.ep_combine(to_dev(rows), wts, None, to_dev(dst), T, H, K, B.EP_BF16, rows.shape[0], out)
        torch.cuda.synchronize()
        got = to_host(out, np.uint16)
        exp = np.array([[int(v, 16) for v in r] for r in c["out_hex"]], np.uint16)
        assert np.array_equal(got[:, :exp.shape[1]], exp), c["name"]
        assert np.all(got[:, exp.shape[1]:] == 0)


def _golden_combine_case(c, fp32):
    """Rows, slots, weights and expected output of one hand-worked combine case."""
    if fp32:
        return (np.array(c["y_rows"], np.float32), np.array(c["dst_slot"], np.int32),
                None if c["topk_weights"] is None else np.array(c["topk_weights"], np.float32),
                np.array(c["out"], np.float32))
    hx = lambda rows: np.array([[int(v, 16) for v in r] for r in rows], np.uint16)  # noqa: E731
    return (hx(c["y_rows_hex"]), np.array(c["dst_slot"], np.int32),
            None if c["topk_weights"] is None else np.array(c["topk_weights"], np.float32),
            hx(c["out_hex"]))


@pytest.mark.parametrize("T,wg_cap", [(5, 0), (1024, 0), (1030, 64)],
                         ids=["sliced_gather", "row_stream", "capped_gather"])
@pytest.mark.parametrize("fp32", [False, True], ids=["bf16", "fp32"])
def test_combine_hand_worked_every_kernel(T, wg_cap, fp32):
    """Every hand-worked combine case (k order, product rounded before the add,
    ties, masking, unit weights) through each combine kernel at hidden 7168:
    a case's channels are repeated across the row and its tokens over T tokens,
    so 5 tokens take the sliced gather, 1024 the row stream and a capped stream
    the gather in 1024-thread workgroups. Expected values are the hand-worked
    ones, bit for bit (both types)."""
    data = json.load(open(os.path.join(GOLDEN, "combine_worked_examples.json")))
    H, dtype = 7168, (B.EP_FP32 if fp32 else B.EP_BF16)
    s = torch.cuda.Stream()
    try:
        B.ep_set_workgroup_limit(s, wg_cap)
        for c in data["combine_f32" if fp32 else "combine"]:
            rows0, dst0, w0, exp0 = _golden_combine_case(c, fp32)
            while not B.ep_supported(2, H, dst0.shape[1], dtype):  # pad with masked entries
                dst0 = np.concatenate([dst0, np.full((dst0.shape[0], 1), -1, np.int32)], axis=1)
                if w0 is not None:
                    w0 = np.concatenate([w0, np.zeros((w0.shape[0], 1), np.float32)], axis=1)
            reps = H // rows0.shape[1]
            rows = np.tile(rows0, (1, reps))
            tok = np.arange(T) % dst0.shape[0]  # token t repeats hand-worked token t mod T0
            dst, K = dst0[tok], dst0.shape[1]
            wts = None if w0 is None else to_dev(w0[tok])
            _say(f"[golden combine] {c['name']} T={T} K={K} cap={wg_cap} fp32={fp32}")
            out = (torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda:0") if fp32
                   else torch.full((T, H), 0x7FC1, dtype=torch.int16, device="cuda:0"))
            y_d, dst_d = to_dev(rows), to_dev(dst)
            torch.cuda.synchronize()  # buffers were filled on the default stream
            B.ep_combine(y_d, wts, None, dst_d, T, H, K, dtype, rows.shape[0], out, s)
            s.synchronize()
            got = to_host(out).view(np.uint32) if fp32 else to_host(out, np.uint16)
            exp = np.tile(exp0, (1, reps))[tok]
            exp = exp.view(np.uint32) if fp32 else exp
            assert np.array_equal(got, exp), c["name"]
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)


def test_combine_rounding_ties_and_specials():
    """Sums that land exactly on bf16 ties, overflow, infinities and NaNs."""
    H, T, K = 1024, 64, 2
    g = np.random.default_rng(5)
    cap = T * K
    y = np.zeros((cap, H), np.uint16)
    m = g.integers(0, 128, (T, H)).astype(np.uint16)
    y[0::2] = 0x3F80 | m                                   # 1 + m/128
    y[1::2] = 0x3B80                                       # 2^-8: every sum is a tie
    y[1::2, :16] = g.integers(0, 0x10000, (T, 16)).astype(np.uint16)  # random bits incl. inf / NaN
    y[0::2, 16] = 0x7F7F                                   # max finite + max finite -> inf
    y[1::2, 16] = 0x7F7F
    y[0::2, 17] = 0x7F80                                   # +inf + -inf -> NaN
    y[1::2, 17] = 0xFF80
    dst = np.arange(cap, dtype=np.int32).reshape(T, K)
    out = torch.zeros((T, H), dtype=torch.int16, device="cuda:0")
    B.ep_combine(to_dev(y), None, None, to_dev(dst), T, H, K, B.EP_BF16, cap, out)
    torch.cuda.synchronize()
    got = to_host(out, np.uint16)
    ref = oracle.combine(y, dst, None)
    nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    nan_r = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    assert np.array_equal(nan_g, nan_r), "NaN positions"
    assert np.array_equal(got[~nan_r], ref[~nan_r]), "non-NaN results bit-exact"
    assert np.all(got[:, 16] == 0x7F80)


DTYPES = [
    # T, H, E, K, A, dtype, scales, combine dtype
    (700, 1024, 64, 8, 4, I.FP32, False, I.FP32),
    (513, 3584, 256, 8, 1, I.FP4X2, True, I.BF16),    # 7168 e2m1 values + 56 scales per token
    (300, 256, 32, 4, 2, I.FP4X2, False, I.BF16),
    (1000, 7168, 128, 6, 16, I.FP8_E4M3, False, I.BF16),
    (2049, 7168, 256, 8, 128, I.BF16, False, I.FP32),  # fp32 combine at the full hidden size
    (40, 2048, 16, 1, 1, I.FP32, False, I.FP32),
]


@pytest.mark.parametrize("T,H,E,K,A,dtype,scales,out_dtype", DTYPES)
def test_dtype_variants(T, H, E, K, A, dtype, scales, out_dtype):
    """fp32 / fp4x2 / scale-less fp8 dispatch and fp32 combine against the oracle."""
    w = I.custom(f"d{dtype}_{T}_{H}", 3000 + T, T, H, E, K, A, dtype, "uniform",
                 out_dtype=out_dtype, scales=scales)
    _say(f"[dtype] {w}")
    case = I.make_case(w, mask_frac=0.03)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case)
    dc.layout()
    dc.dispatch()
    out = dc.combine()
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])
    if out_dtype == I.FP32:
        got = to_host(out)
        exp = oracle.combine_f32(case.y, ref["dst_slot"], case.topk_weights)
        assert np.array_equal(np.isnan(got), np.isnan(exp))
        same = got.view(np.uint32) == exp.view(np.uint32)
        _say(f"combine fp32: {int(same.sum())}/{same.size} bit-exact")
        assert same.all(), "fp32 combine differs from the oracle's binary32 arithmetic"
    else:
        check_combine(to_host(out, np.uint16), oracle.combine(case.y, ref["dst_slot"], case.topk_weights),
                      w.name)


def test_combine_with_bias():
    """Combine adds a per-token bias once, after the k-order sum (bf16 and fp32)."""
    data = json.load(open(os.path.join(GOLDEN, "combine_worked_examples.json")))
    c = data["combine_bias"][0]
    H = 256
    rows = np.zeros((2, H), np.uint16)
    bias = np.zeros((1, H), np.uint16)
    for r, row in enumerate(c["y_rows_hex"]):
        rows[r, :8] = [int(v, 16) for v in row]
    bias[0, :8] = [int(v, 16) for v in c["bias_hex"][0]]
    dst = np.array([[0, 1]], np.int32)
    out = torch.zeros((1, H), dtype=torch.int16, device="cuda:0")
    B.ep_combine(to_dev(rows), None, to_dev(bias), to_dev(dst), 1, H, 2, B.EP_BF16, 2, out)
    torch.cuda.synchronize()
    got = to_host(out, np.uint16)
    assert np.array_equal(got[0, :8], [int(v, 16) for v in c["out_hex"][0]])
    for out_dtype in (I.BF16, I.FP32):
        w = I.custom(f"bias{out_dtype}", 61, 1500, 2048, 64, 8, 2, I.BF16, "uniform",
                     out_dtype=out_dtype)
        case = I.make_case(w, mask_frac=0.02)
        ref = oracle.layout(case.topk_idx, w.E, w.A)
        dc = DeviceCase(case)
        dc.layout()
        if out_dtype == I.BF16:
            bias = I.normal_bf16(w.seed, 9, w.T, w.H)
            out = dc.combine(bias=to_dev(bias))
            torch.cuda.synchronize()
            check_combine(to_host(out, np.uint16),
                          oracle.combine(case.y, ref["dst_slot"], case.topk_weights, bias), "bias")
        else:
            bias = I.normal_f32(w.seed, 9, w.T, w.H)
            out = dc.combine(bias=to_dev(bias))
            torch.cuda.synchronize()
            exp = oracle.combine_f32(case.y, ref["dst_slot"], case.topk_weights, bias)
            assert np.array_equal(to_host(out).view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("name", ["prefill_aligned", "mori_default"])
def test_graph_capture_replay(name):
    """layout -> dispatch -> combine captured into one HIP graph (nothing on the path allocates,
    synchronises or records a memset); every replay, with eager steps in between, matches eager."""
    w = I.WORKLOADS[name]
    case = I.make_case(w)
    dev = "cuda:0"
    idx, wts, x, y = to_dev(case.topk_idx), to_dev(case.topk_weights), to_dev(case.x), to_dev(case.y)
    counts = torch.zeros(w.E, dtype=torch.int32, device=dev)
    offs = torch.zeros(w.E + 1, dtype=torch.int32, device=dev)
    dst = torch.zeros((w.T, w.K), dtype=torch.int32, device=dev)
    meta = torch.zeros((w.T, w.K + 2), dtype=torch.int32, device=dev)
    nrecv = torch.zeros(1, dtype=torch.int32, device=dev)
    wsb = B.ep_layout_workspace_bytes(w.T, w.K, w.E)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    X = torch.zeros((w.cap, w.H), dtype=torch.int16, device=dev)
    out = torch.zeros((w.T, w.H), dtype=torch.int16, device=dev)

    def step(stream):
        B.ep_layout(idx, w.T, w.K, w.E, w.A, w.cap, counts, offs, dst, meta, nrecv, ws, wsb, stream)
        B.ep_dispatch(x, None, None, dst, w.T, w.H, w.K, B.EP_BF16, w.cap, X, None, None, stream)
        B.ep_combine(y, wts, None, dst, w.T, w.H, w.K, B.EP_BF16, w.cap, out, stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = (counts, offs, dst, meta, nrecv, X, out)
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(4):
        for t in outs:
            t.zero_()  # a fill kernel outside the graph, so every replay must rewrite everything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {r} differs from eager"
        step(torch.cuda.current_stream())  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("path", ["expand", "non-expand"])
def test_graph_capture_replay_one_launch_calls(path):
    """A decode step through the one-launch layout + dispatch calls (ep_layout_dispatch, or
    ep_layout_dispatch_compact) and combine, captured into one HIP graph; every replay, with
    eager steps in between, matches eager."""
    w = I.WORKLOADS["decode_zipf"]
    case = I.make_case(w)
    dev = "cuda:0"
    T, K, E, H = w.T, w.K, w.E, w.H
    idx, wts, x = to_dev(case.topk_idx), to_dev(case.topk_weights), to_dev(case.x)
    y = to_dev(case.y) if path == "expand" else to_dev(case.y[:T])
    counts = torch.zeros(E, dtype=torch.int32, device=dev)
    offs = torch.zeros(E + 1, dtype=torch.int32, device=dev)
    dst = torch.zeros((T, K), dtype=torch.int32, device=dev)
    meta = torch.zeros((T, K + 2), dtype=torch.int32, device=dev)
    nrecv = torch.zeros(1, dtype=torch.int32, device=dev)
    wsb = B.ep_layout_workspace_bytes(T, K, E)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
    rows = w.cap if path == "expand" else T
    X = torch.zeros((rows, H), dtype=torch.int16, device=dev)
    Xw = torch.zeros((rows,), dtype=torch.float32, device=dev)
    recv_i = torch.zeros((T, K), dtype=torch.int32, device=dev)
    recv_w = torch.zeros((T, K), dtype=torch.float32, device=dev)
    out = torch.zeros((T, H), dtype=torch.int16, device=dev)

    def step(stream):
        if path == "expand":
            B.ep_layout_dispatch(idx, T, K, E, w.A, w.cap, counts, offs, dst, meta, nrecv, ws, wsb,
                                 x, None, wts, H, B.EP_BF16, X, None, Xw, stream)
            B.ep_combine(y, wts, None, dst, T, H, K, B.EP_BF16, w.cap, out, stream)
        else:
            B.ep_layout_dispatch_compact(idx, T, K, E, w.A, w.cap, counts, offs, dst, meta, nrecv,
                                         ws, wsb, x, None, wts, H, B.EP_BF16, X, None, recv_i,
                                         recv_w, stream)
            B.ep_combine_compact(y, None, dst, meta, nrecv, T, H, K, B.EP_BF16, out, stream)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = (counts, offs, dst, meta, nrecv, X, Xw, recv_i, recv_w, out)
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for r in range(4):
        for t in outs:
            t.zero_()  # a fill kernel outside the graph, so every replay must rewrite everything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a, b), f"replay {r} differs from eager"
        step(torch.cuda.current_stream())  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("T,H,E,K,A,dtype", [(4096, 256, 256, 8, 128, I.BF16),
                                              (700, 512, 64, 4, 16, I.FP8_E4M3),
                                              (300, 1024, 16, 2, 1, I.BF16)])
def test_zero_padding_after_dispatch(T, H, E, K, A, dtype):
    """Whole expand buffers (rows, scale rows, weights) match the oracle after dispatch + zero-fill."""
    w = I.custom(f"zp{T}", 4000 + T, T, H, E, K, A, dtype, "uniform")
    case = I.make_case(w, with_y=False)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    dc.layout()
    dc.dispatch()
    S = 0 if dc.expand_s is None else dc.expand_s.shape[1]
    B.ep_zero_padding(dc.expand_x, dc.row_bytes, dc.expand_s, S, dc.expand_w, dc.lay["counts"],
                      dc.lay["offsets"], w.E, w.A, w.cap)
    torch.cuda.synchronize()
    X = np.full((w.cap, dc.row_bytes), dc.sentinel, np.uint8)
    Xs = None if S == 0 else np.full((w.cap, S), -3.0, np.float32)
    Xw = np.full(w.cap, -5.0, np.float32)
    oracle.dispatch(case.x, ref["dst_slot"], w.cap, x_scales=case.x_scales,
                    topk_weights=case.topk_weights, expand_x=X, expand_scales=Xs, expand_weights=Xw)
    oracle.zero_padding(X, ref["counts"], ref["offsets"], Xs, Xw)
    assert np.array_equal(to_host(dc.expand_x), X)
    assert np.array_equal(to_host(dc.expand_w).view(np.uint32), Xw.view(np.uint32))
    if Xs is not None:
        assert np.array_equal(to_host(dc.expand_s).view(np.uint32), Xs.view(np.uint32))
