"""CU-limited mode on the GPU: results under a workgroup cap equal the oracle's.

Source: "MORI JIT v2" section 5.1 (geometry buckets; fewer workgroups leave
compute units to the expert GEMM; never more workgroups than compute units)
and the EpCfg default of 64 workgroups; DeepEP overall architecture (a few
SMs for communication). A cap changes only the launch geometry (workgroups
of 1024 or 512 threads whose waves, or layout tiles, loop), so every output
must be bit-identical to the oracle's, as without a cap.
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
from tests.gpu_util import DEV, DeviceCase, layout_to_host, to_dev, to_host  # noqa: E402


def _say(msg):
    print(msg, flush=True)


@pytest.fixture
def capped_stream():
    s = torch.cuda.Stream()
    yield s
    torch.cuda.synchronize()
    B.ep_set_workgroup_limit(s, 0)


def test_cap_is_clamped_and_cleared(capped_stream):
    s = capped_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B.ep_set_workgroup_limit(s, 64)
    assert B.ep_get_workgroup_limit(s) == 64
    B.ep_set_workgroup_limit(s, 100000)
    assert B.ep_get_workgroup_limit(s) == cus
    assert B.ep_get_workgroup_limit(torch.cuda.current_stream()) == 0  # other streams untouched
    B.ep_set_workgroup_limit(s, 0)
    assert B.ep_get_workgroup_limit(s) == 0


CASES = [
    # name, T, H, E, K, A, dtype, mask, cap: layout takes all three launch shapes
    ("prefill two-launch layout", 4096, 7168, 256, 8, 128, I.BF16, 0.0, 64),
    ("two-launch layout, tiles loop", 4096, 7168, 256, 8, 128, I.BF16, 0.2, 7),
    ("fused layout, tiles loop", 1500, 1024, 256, 8, 16, I.BF16, 0.1, 5),
    ("single tile, one workgroup", 100, 2048, 64, 8, 1, I.BF16, 0.0, 1),
    ("fp8 with scales", 2048, 7168, 256, 8, 1, I.FP8_E4M3, 0.0, 32),
    ("fp32 rows, fp32 combine", 777, 256, 32, 6, 4, I.FP32, 0.3, 3),
    ("fp32 rows of 28 chunks per lane, pieces", 1200, 7168, 64, 8, 1, I.FP32, 0.1, 16),
    ("tile-scan layout, tiles loop", 20000, 256, 1024, 8, 4, I.BF16, 0.05, 6),
]


@pytest.mark.parametrize("name,T,H,E,K,A,dtype,mask,cap", CASES)
def test_capped_path_matches_oracle(capped_stream, name, T, H, E, K, A, dtype, mask, cap):
    s = capped_stream
    _say(f"cap {cap}: {name} T={T} H={H} E={E} K={K} A={A} dtype={dtype} mask={mask}")
    B.ep_set_workgroup_limit(s, cap)
    out_dtype = I.FP32 if dtype == I.FP32 else I.BF16
    w = I.custom(f"cap_{T}_{cap}", 700 + cap, T, H, E, K, A, dtype, out_dtype=out_dtype)
    case = I.make_case(w, mask_frac=mask)
    with torch.cuda.stream(s):
        dc = DeviceCase(case)
        lay = dc.layout(stream=s)
        dc.dispatch(stream=s)
        out = dc.combine(stream=s)
        B.ep_zero_padding(dc.expand_x, dc.row_bytes, dc.expand_s,
                          0 if dc.expand_s is None else dc.expand_s.shape[1], dc.expand_w,
                          lay["counts"], lay["offsets"], E, A, w.cap, s)
    s.synchronize()

    ref = oracle.layout(case.topk_idx, E, A)
    got = layout_to_host(lay)
    for k in ("counts", "offsets", "dst_slot"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["num_recv"] == ref["num_recv"]
    assert np.array_equal(got["recv_src_metadata"], ref["recv_src_metadata"])

    # whole expand buffers: dispatch then zero-fill of padding, rows past offsets[E] untouched
    ex = np.full((w.cap, dc.row_bytes), dc.sentinel, np.uint8)
    es = (np.full((w.cap, case.x_scales.shape[1]), -3.0, np.float32)
          if dc.expand_s is not None else None)
    ew = np.full((w.cap,), -5.0, np.float32)
    oracle.dispatch(case.x, ref["dst_slot"], w.cap, x_scales=case.x_scales,
                    topk_weights=case.topk_weights, expand_x=ex, expand_scales=es, expand_weights=ew)
    oracle.zero_padding(ex, ref["counts"], ref["offsets"], es, ew)
    assert np.array_equal(to_host(dc.expand_x), ex), "expand_x"
    assert np.array_equal(to_host(dc.expand_w).view(np.uint32), ew.view(np.uint32)), "expand_weights"
    if es is not None:
        assert np.array_equal(to_host(dc.expand_s).view(np.uint32), es.view(np.uint32)), "scales"

    if out_dtype == I.FP32:
        want = oracle.combine_f32(case.y, ref["dst_slot"], case.topk_weights)
        assert np.array_equal(to_host(out).view(np.uint32), want.view(np.uint32)), "combine"
    else:
        want = oracle.combine(case.y, ref["dst_slot"], case.topk_weights)
        d = pins.bf16_ulp_distance(to_host(out, np.uint16), want)
        _say(f"  combine exact={np.mean(d == 0):.6f} max_ulp={int(d.max())}")
        assert d.max() <= 1


@pytest.mark.parametrize("cap", [1, 16])
def test_capped_non_expand_matches_oracle(capped_stream, cap):
    s = capped_stream
    w = I.custom(f"cap_ne_{cap}", 900 + cap, 3000, 7168, 256, 8, 128)
    _say(f"cap {cap}: non-expand T={w.T}")
    B.ep_set_workgroup_limit(s, cap)
    case = I.make_case(w, with_y=False, mask_frac=0.3)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    n = ref["num_recv"]
    with torch.cuda.stream(s):
        dc = DeviceCase(case, with_y=False)
        lay = dc.layout(stream=s)
        recv_x = torch.full((w.T, dc.row_bytes), 0x5A, dtype=torch.uint8, device=DEV)
        recv_i = torch.full((w.T, w.K), -7, dtype=torch.int32, device=DEV)
        recv_w = torch.full((w.T, w.K), -5.0, dtype=torch.float32, device=DEV)
        B.ep_dispatch_compact(dc.x, None, dc.idx, dc.wts, lay["dst_slot"], lay["meta"],
                              lay["num_recv"], w.T, w.H, w.K, w.dtype, recv_x, None, recv_i,
                              recv_w, s)
        y = I.normal_bf16(w.seed, 4, w.T, w.H)
        bias = I.normal_bf16(w.seed, 9, w.T, w.H)
        out = torch.empty((w.T, w.H), dtype=torch.int16, device=DEV)
        B.ep_combine_compact(to_dev(y), to_dev(bias), lay["dst_slot"], lay["meta"],
                             lay["num_recv"], w.T, w.H, w.K, B.EP_BF16, out, s)
    s.synchronize()
    rx, _, ri, rw = oracle.dispatch_compact(case.x, case.topk_idx, ref["dst_slot"],
                                            ref["recv_src_metadata"], n, None, case.topk_weights)
    gx = to_host(recv_x)
    assert np.array_equal(gx[:n], rx) and np.all(gx[n:] == 0x5A)
    assert np.array_equal(to_host(recv_i)[:n], ri)
    assert np.array_equal(to_host(recv_w)[:n].view(np.uint32), rw.view(np.uint32))
    want = oracle.combine_compact(y, ref["dst_slot"], ref["recv_src_metadata"], n, bias)
    assert pins.bf16_ulp_distance(to_host(out, np.uint16), want).max() <= 1
    # binary32 rows under the same cap
    yf, bf = I.normal_f32(w.seed, 4, w.T, w.H), I.normal_f32(w.seed, 9, w.T, w.H)
    yf_d, bf_d = to_dev(yf), to_dev(bf)
    out32 = torch.empty((w.T, w.H), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    B.ep_combine_compact(yf_d, bf_d, lay["dst_slot"], lay["meta"], lay["num_recv"], w.T, w.H, w.K,
                         B.EP_FP32, out32, s)
    s.synchronize()
    want32 = oracle.combine_compact_f32(yf, ref["dst_slot"], ref["recv_src_metadata"], n, bf)
    assert np.array_equal(to_host(out32).view(np.uint32), want32.view(np.uint32))


def test_two_host_threads_two_streams_two_caps():
    """Two host threads call the library at the same time, each on its own
    stream with its own workgroup cap (none and 64) and its own buffers; the
    caps are per stream and every call's state is its own, so both end with
    the oracle's results."""
    import threading
    runs = []
    for i, (T, cap) in enumerate([(3000, 0), (2000, 64)]):
        w = I.custom(f"threads{i}", 9700 + i, T, 2048, 64, 8, 4)
        case = I.make_case(w, mask_frac=0.1)
        runs.append({"w": w, "case": case, "dc": DeviceCase(case), "cap": cap,
                     "stream": torch.cuda.Stream()})
    torch.cuda.synchronize()
    errors = []

    def drive(r):
        s = r["stream"]
        try:
            B.ep_set_workgroup_limit(s, r["cap"])  # raises EpError on failure
            assert B.ep_get_workgroup_limit(s) == r["cap"]
            with torch.cuda.stream(s):
                for _ in range(10):
                    r["lay"] = r["dc"].layout(stream=s, plan=True)
                    r["dc"].dispatch(stream=s, plan=True)
                    r["out"] = r["dc"].combine(stream=s)
            s.synchronize()
        except Exception as e:  # reported below, on the test's own thread
            errors.append(e)

    threads = [threading.Thread(target=drive, args=(r,)) for r in runs]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    for r in runs:
        B.ep_set_workgroup_limit(r["stream"], 0)
    assert not errors, errors

    for r in runs:
        w, case, dc = r["w"], r["case"], r["dc"]
        _say(f"thread run: T={w.T} cap={r['cap']}")
        ref = oracle.layout(case.topk_idx, w.E, w.A)
        got = layout_to_host(r["lay"])
        for k in ("counts", "offsets", "dst_slot"):
            assert np.array_equal(got[k], ref[k]), k
        assert np.array_equal(got["recv_src_metadata"], ref["recv_src_metadata"])
        ex = np.full((w.cap, dc.row_bytes), dc.sentinel, np.uint8)
        ew = np.full((w.cap,), -5.0, np.float32)
        oracle.dispatch(case.x, ref["dst_slot"], w.cap, topk_weights=case.topk_weights,
                        expand_x=ex, expand_weights=ew)
        assert np.array_equal(to_host(dc.expand_x), ex), "expand_x"
        assert np.array_equal(to_host(dc.expand_w).view(np.uint32), ew.view(np.uint32))
        want = oracle.combine(case.y, ref["dst_slot"], case.topk_weights)
        assert pins.bf16_ulp_distance(to_host(r["out"], np.uint16), want).max() <= 1
