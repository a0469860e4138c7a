"""Non-expand dispatch / combine on the GPU vs the CPU oracle, through the C ABI.

Source: DeepEP overall-architecture page, EPHandle do_expand = false (one
row per received token; recv_x, recv_topk_idx, recv_topk_weights) and the
combine reduce epilogue with bias. Bar: received rows, scale rows, ids and
weights bit-exact; combine within 1 bf16 ulp (one binary32 add then RNE on
both sides, so the test also reports exact matches). Rows past num_recv
must stay untouched.
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
from tests.gpu_util import DEV, dev_layout, layout_to_host, to_dev, to_host  # noqa: E402

ELT = {I.BF16: 2, I.FP32: 4, I.FP8_E4M3: 1, I.FP4X2: 1}


def _say(msg):
    print(msg, flush=True)


def _run(w: I.Workload, mask: float = 0.0, weights: bool = True, bias: bool = True,
         oob_every: int = 0, combine_fp32: bool = False):
    """Layout -> non-expand dispatch -> non-expand combine on the GPU, each checked."""
    _say(f"non-expand {w.name}: T={w.T} H={w.H} E={w.E} K={w.K} A={w.A} dtype={w.dtype} "
         f"mask={mask} weights={weights} bias={bias}")
    case = I.make_case(w, with_y=False, mask_frac=mask)
    if oob_every:
        case.topk_idx[::oob_every, -1] = w.E + 5  # ids outside [0, E) are masked like -1
    T, K = w.T, w.K
    idx_d, wts_d, x_d = to_dev(case.topk_idx), to_dev(case.topk_weights), to_dev(case.x)
    xs_d = to_dev(case.x_scales) if case.x_scales is not None else None
    lay = dev_layout(idx_d, T, K, w.E, w.A, w.cap)
    got_lay = layout_to_host(lay)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    assert np.array_equal(got_lay["dst_slot"], ref["dst_slot"]) and got_lay["num_recv"] == ref["num_recv"]
    assert np.array_equal(got_lay["recv_src_metadata"], ref["recv_src_metadata"])
    n = ref["num_recv"]

    row_bytes = w.H * ELT[w.dtype]
    rows = max(T, 1)
    recv_x = torch.full((rows, row_bytes), 0x5A, dtype=torch.uint8, device=DEV)
    recv_s = (torch.full((rows, case.x_scales.shape[1]), -3.0, dtype=torch.float32, device=DEV)
              if xs_d is not None else None)
    recv_i = torch.full((rows, K), -7, dtype=torch.int32, device=DEV)
    recv_w = torch.full((rows, K), -5.0, dtype=torch.float32, device=DEV) if weights else None
    B.ep_dispatch_compact(x_d, xs_d, idx_d, wts_d if weights else None, lay["dst_slot"], lay["meta"],
                          lay["num_recv"], T, w.H, K, w.dtype, recv_x, recv_s, recv_i, recv_w)
    torch.cuda.synchronize()

    rx, rs, ri, rw = oracle.dispatch_compact(case.x, case.topk_idx, ref["dst_slot"],
                                             ref["recv_src_metadata"], n, case.x_scales,
                                             case.topk_weights if weights else None)
    gx, gi = to_host(recv_x), to_host(recv_i)
    assert np.array_equal(gx[:n], rx), "recv_x"
    assert np.all(gx[n:] == 0x5A), "rows past num_recv were written"
    assert np.array_equal(gi[:n], ri), "recv_topk_idx"
    assert np.all(gi[n:] == -7)
    if recv_s is not None:
        gs = to_host(recv_s)
        assert np.array_equal(gs[:n].view(np.uint8), rs), "recv_scales"
        assert np.all(gs[n:] == -3.0)
    if weights:
        gw = to_host(recv_w)
        assert np.array_equal(gw[:n].view(np.uint32), rw.view(np.uint32)), "recv_topk_weights"
        assert np.all(gw[n:] == -5.0)

    H_out = 2 * w.H if w.dtype == I.FP4X2 else w.H
    if combine_fp32:  # the expert side hands back one binary32 row per received token
        y = I.normal_f32(w.seed, 4, rows, H_out)
        b = I.normal_f32(w.seed, 9, rows, H_out)[:T] if bias else None
        out = torch.full((rows, H_out), float("nan"), dtype=torch.float32, device=DEV)
        B.ep_combine_compact(to_dev(y), to_dev(b) if bias else None, lay["dst_slot"], lay["meta"],
                             lay["num_recv"], T, H_out, K, B.EP_FP32, out)
        torch.cuda.synchronize()
        got = to_host(out)[:T]
        want = oracle.combine_compact_f32(y, ref["dst_slot"], ref["recv_src_metadata"], n, b)
        same = got.view(np.uint32) == want.view(np.uint32)
        _say(f"  num_recv={n} fp32 combine bit-exact {int(same.sum())}/{same.size}")
        assert same.all(), "fp32 non-expand combine differs from the oracle"
        return case, ref, recv_x, n
    # combine: the expert side hands back one bf16 row per received token
    y = I.normal_bf16(w.seed, 4, rows, H_out)
    b = I.normal_bf16(w.seed, 9, rows, H_out)[:T] if bias else None
    out = torch.full((rows, H_out), 0x7FC1, dtype=torch.int16, device=DEV)
    B.ep_combine_compact(to_dev(y), to_dev(b) if bias else None, lay["dst_slot"], lay["meta"],
                         lay["num_recv"], T, H_out, K, B.EP_BF16, out)
    torch.cuda.synchronize()
    got = to_host(out, np.uint16)[:T]
    want = oracle.combine_compact(y, ref["dst_slot"], ref["recv_src_metadata"], n, b)
    d = pins.bf16_ulp_distance(got, want)
    _say(f"  num_recv={n} combine exact={np.mean(d == 0):.6f} max_ulp={int(d.max()) if d.size else 0}")
    assert d.size == 0 or d.max() <= 1, "combine beyond 1 bf16 ulp"
    if not bias:
        assert np.array_equal(got, want), "without a bias rows come back bit for bit"
    return case, ref, recv_x, n


@pytest.mark.parametrize("name", ["prefill_aligned", "mori_default", "decode_zipf", "fp8_hot8"])
def test_workload_full_size(name):
    _run(I.WORKLOADS[name])


def test_fp4x2_rows_with_scales():
    _run(I.EXTRA_WORKLOADS["prefill_fp4x2"], mask=0.2)


RAGGED = [
    # T, H, E, K, A, dtype, mask, weights, bias
    (1, 256, 8, 1, 1, I.BF16, 0.0, True, True),
    (333, 520, 32, 4, 16, I.BF16, 0.3, True, True),     # 65 chunks per row: a one-chunk tail slice
    (777, 7168, 256, 8, 128, I.BF16, 0.9, False, True),  # many tokens receive nothing
    (1000, 104, 64, 6, 1, I.FP32, 0.25, True, False),     # fp32 rows move unchanged, 416 bytes
    (513, 1024, 16, 2, 4, I.FP8_E4M3, 0.5, True, True),
    (64, 7168, 256, 8, 1, I.BF16, 0.0, True, False),
]


@pytest.mark.parametrize("T,H,E,K,A,dtype,mask,weights,bias", RAGGED)
def test_ragged_shapes(T, H, E, K, A, dtype, mask, weights, bias):
    w = I.custom(f"ne_{T}_{H}_{K}", 500 + T, T, H, E, K, A, dtype)
    _run(w, mask=mask, weights=weights, bias=bias, oob_every=5)


FP32_COMBINE = [
    # T, H, E, K, A, dtype, mask, bias: binary32 rows through the non-expand combine
    (4096, 7168, 256, 8, 128, I.BF16, 0.0, True),    # the prefill shape, 28 KiB rows
    (333, 520, 32, 4, 16, I.BF16, 0.3, True),         # 130 chunks per row: a two-chunk tail slice
    (777, 1024, 256, 8, 1, I.FP8_E4M3, 0.9, False),   # many tokens receive nothing; no bias
    (1, 256, 8, 1, 1, I.BF16, 0.0, True),
]


@pytest.mark.parametrize("T,H,E,K,A,dtype,mask,bias", FP32_COMBINE)
def test_combine_fp32_rows(T, H, E, K, A, dtype, mask, bias):
    w = I.custom(f"ne32_{T}_{H}", 900 + T, T, H, E, K, A, dtype)
    _run(w, mask=mask, bias=bias, oob_every=7, combine_fp32=True)


def test_nothing_received():
    w = I.custom("ne_none", 7, 200, 256, 16, 4, 2)
    _, ref, _, n = _run(w, mask=1.0)
    assert n == 0 and ref["num_recv"] == 0


def test_empty_input():
    z = torch.zeros(16, dtype=torch.int32, device=DEV)
    B.ep_dispatch_compact(None, None, None, None, None, None, z, 0, 256, 8, B.EP_BF16, None, None,
                          None, None)
    B.ep_combine_compact(None, None, None, None, z, 0, 256, 8, B.EP_BF16, None)
    torch.cuda.synchronize()


def test_round_trip_returns_x():
    """Combining the received rows unchanged gives x back for every received token."""
    w = I.custom("ne_rt", 33, 2048, 7168, 256, 8, 128)
    case, ref, recv_x, n = _run(w, mask=0.3, bias=False)
    T = w.T
    out = torch.full((T, w.H), 0x7FC1, dtype=torch.int16, device=DEV)
    lay = dev_layout(to_dev(case.topk_idx), T, w.K, w.E, w.A, w.cap)
    B.ep_combine_compact(recv_x, None, lay["dst_slot"], lay["meta"], lay["num_recv"], T, w.H, w.K,
                         B.EP_BF16, out)
    got = to_host(out, np.uint16)
    recv = (ref["dst_slot"] >= 0).any(axis=1)
    assert np.array_equal(got[recv], case.x[recv]) and np.all(got[~recv] == 0)


FUSED = [
    # T, H, E, K, A, mask, dtype, scales, routing, workgroup cap: one tile runs layout and the
    # non-expand dispatch as one launch; larger batches fall back to two launches
    (128, 7168, 256, 8, 1, 0.0, I.BF16, False, "zipf", 0),       # the decode shape
    (64, 256, 16, 2, 1, 0.2, I.BF16, False, "uniform", 0),       # tiny, with masking
    (100, 7168, 256, 8, 128, 0.1, I.FP8_E4M3, True, "uniform", 0),
    (100, 3584, 128, 8, 4, 0.05, I.FP4X2, True, "uniform", 0),
    (50, 1024, 32, 4, 2, 0.2, I.FP32, False, "uniform", 0),
    (170, 2048, 64, 6, 4, 0.1, I.BF16, False, "uniform", 0),     # 1020 entries, K = 6
    (64, 512, 300, 8, 1, 0.0, I.BF16, False, "uniform", 0),      # 512-entry tile
    (32, 512, 1024, 8, 3, 0.5, I.BF16, False, "uniform", 0),     # 256-entry tile
    (1, 7168, 64, 8, 1, 0.0, I.BF16, False, "uniform", 0),       # one token
    (128, 7168, 256, 8, 1, 0.1, I.BF16, False, "zipf", 3),       # capped
    (3000, 2048, 256, 8, 16, 0.05, I.BF16, False, "uniform", 0),  # several tiles: two launches
]


@pytest.mark.parametrize("weights", [True, False])
@pytest.mark.parametrize("T,H,E,K,A,mask,dtype,scales,routing,cap", FUSED)
def test_layout_dispatch_compact(T, H, E, K, A, mask, dtype, scales, routing, cap, weights):
    """ep_layout_dispatch_compact produces what ep_layout and ep_dispatch_compact produce."""
    w = I.custom(f"nefused{T}_{E}_{K}", 9800 + T + E, T, H, E, K, A, dtype, routing,
                 scales=scales)
    _say(f"[layout + non-expand dispatch] {w} cap {cap} weights {weights}")
    case = I.make_case(w, with_y=False, mask_frac=mask)
    case.topk_idx[::7, 0] = w.E + 5  # ids outside [0, E) are masked like -1
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    n = ref["num_recv"]
    idx_d, wts_d, x_d = to_dev(case.topk_idx), to_dev(case.topk_weights), to_dev(case.x)
    xs_d = to_dev(case.x_scales) if case.x_scales is not None else None
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    dst = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    meta = torch.full((T, K + 2), -7, dtype=torch.int32, device=DEV)
    nrecv = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    wsb = B.ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    row_bytes = H * ELT[dtype]
    recv_x = torch.full((T, row_bytes), 0x5A, dtype=torch.uint8, device=DEV)
    recv_s = (torch.full((T, case.x_scales.shape[1]), -3.0, dtype=torch.float32, device=DEV)
              if xs_d is not None else None)
    recv_i = torch.full((T, K), -7, dtype=torch.int32, device=DEV)
    recv_w = torch.full((T, K), -5.0, dtype=torch.float32, device=DEV) if weights else None
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # the inputs and buffers were written there
    try:
        B.ep_set_workgroup_limit(s, cap)
        with torch.cuda.stream(s):
            B.ep_layout_dispatch_compact(idx_d, T, K, E, A, w.cap, counts, offsets, dst, meta,
                                         nrecv, ws, wsb, x_d, xs_d, wts_d if weights else None,
                                         H, dtype, recv_x, recv_s, recv_i, recv_w, s)
        s.synchronize()
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)

    got = layout_to_host({"counts": counts, "offsets": offsets, "dst_slot": dst, "meta": meta,
                          "num_recv": nrecv})
    for k in ("counts", "offsets", "dst_slot"):
        assert np.array_equal(got[k], ref[k]), k
    assert got["num_recv"] == n
    assert np.array_equal(got["recv_src_metadata"], ref["recv_src_metadata"])
    rx, rs, ri, rw = oracle.dispatch_compact(case.x, case.topk_idx, ref["dst_slot"],
                                             ref["recv_src_metadata"], n, case.x_scales,
                                             case.topk_weights if weights else None)
    gx, gi = to_host(recv_x), to_host(recv_i)
    assert np.array_equal(gx[:n], rx), "recv_x"
    assert np.all(gx[n:] == 0x5A), "rows past num_recv were written"
    assert np.array_equal(gi[:n], ri), "recv_topk_idx"
    assert np.all(gi[n:] == -7)
    if recv_s is not None:
        gs = to_host(recv_s)
        assert np.array_equal(gs[:n].view(np.uint8), rs), "recv_scales"
        assert np.all(gs[n:] == -3.0)
    if weights:
        gw = to_host(recv_w)
        assert np.array_equal(gw[:n].view(np.uint32), rw.view(np.uint32)), "recv_topk_weights"
        assert np.all(gw[n:] == -5.0)


def test_layout_dispatch_compact_empty():
    """No tokens: the layout's outputs are zero and no received row is written."""
    E, K, H = 256, 8, 7168
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    nrecv = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    recv_x = torch.full((4, 2 * H), 0x5A, dtype=torch.uint8, device=DEV)
    recv_i = torch.full((4, K), -7, dtype=torch.int32, device=DEV)
    B.ep_layout_dispatch_compact(None, 0, K, E, 1, 0, counts, offsets, None, None, nrecv, ws,
                                 B.ep_layout_workspace_bytes(0, K, E), None, None, None, H,
                                 B.EP_BF16, recv_x, None, recv_i, None)
    torch.cuda.synchronize()
    assert np.all(to_host(counts) == 0) and np.all(to_host(offsets) == 0)
    assert int(nrecv.item()) == 0
    assert np.all(to_host(recv_x) == 0x5A) and np.all(to_host(recv_i) == -7)
