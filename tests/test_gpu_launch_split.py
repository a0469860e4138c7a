"""Inputs split over several launches, on a test build with a small launch limit.

The uncapped one-unit-per-wave kernels (the planned and grouped dispatch, the
sliced combine, the non-expand dispatch and combine) take at most 2^26 - 64
units per launch, so
batches past that size run as several launches from a unit offset, or, on
the non-expand path, as one launch of the looping kernel. No test input is
that large. libep_mi355x_small_launch.so is the same library built with the
limit at 4160 units (combine_ep_layout_amd/build.py, build_small_launch),
so these moderate batches run those paths; every output is checked against
the CPU oracle as in the other parity tests.
"""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - only on CPU hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
from combine_ep_layout_amd import binding as B  # noqa: E402
from combine_ep_layout_amd import build as hip_build  # noqa: E402
from combine_ep_layout_amd import inputs as I  # noqa: E402
from tests import pins  # noqa: E402
from tests.gpu_util import DeviceCase, layout_to_host, to_host  # noqa: E402
from tests.test_gpu_non_expand import _run  # noqa: E402
from tests.test_gpu_parity import check_dispatch, check_layout  # noqa: E402

LIMIT = hip_build.SMALL_LAUNCH_UNITS


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def small_launch_library():
    path = hip_build.SMALL_LAUNCH_LIB
    if not os.path.exists(path):  # a test build: its absence skips these tests, not the suite
        pytest.skip(f"{path} is missing: build it with __graft_entry__.build()")
    torch.cuda.synchronize()
    B.use_library(path)
    yield
    torch.cuda.synchronize()
    B.use_library(None)


SPLIT_DISPATCH = [
    # T, H, E, K, A, mask, dtype, scales; units = T * K * slices
    (300, 7168, 256, 8, 128, 0.05, I.BF16, False),   # 33,600 units: 9 launches of 297 entries
    (500, 7168, 64, 6, 1, 0.1, I.FP8_E4M3, True),    # 21,000 units of 7 KiB rows: 6 launches
    (777, 2048, 32, 4, 4, 0.0, I.FP32, False),       # 24,864 units: 6 launches, ragged last
]


@pytest.mark.parametrize("plan", [True, False], ids=["planned", "token-major"])
@pytest.mark.parametrize("T,H,E,K,A,mask,dtype,scales", SPLIT_DISPATCH)
def test_dispatch_over_several_launches(T, H, E, K, A, mask, dtype, scales, plan):
    w = I.custom(f"split{T}_{H}_{K}", 7100 + T, T, H, E, K, A, dtype, "uniform", scales=scales)
    _say(f"[dispatch, launch limit {LIMIT}, plan={plan}] {w}")
    case = I.make_case(w, with_y=False, mask_frac=mask)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    dc.layout(plan=plan)
    dc.dispatch(plan=plan)
    torch.cuda.synchronize()
    check_layout(layout_to_host(dc.lay), ref)
    check_dispatch(dc, ref["dst_slot"])


def test_grouped_dispatch_over_several_launches():
    # x past 128 MiB: groups of 4 entries per wave, 9400 * 2 * 14 = 263,200 units (64 launches)
    w = I.custom("split_grouped", 7300, 9400, 7168, 256, 8, 16, I.BF16, "uniform", scales=False)
    _say(f"[grouped dispatch, launch limit {LIMIT}] {w}")
    case = I.make_case(w, with_y=False, mask_frac=0.03)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case, with_y=False)
    dc.layout()
    dc.dispatch()
    torch.cuda.synchronize()
    check_dispatch(dc, ref["dst_slot"])


@pytest.mark.parametrize("T,H,E,K,A,mask,out_dtype", [
    (1000, 7168, 256, 8, 1, 0.2, I.BF16),    # 7,000 units of 2 KiB slices: 2 launches
    (1023, 7168, 64, 6, 4, 0.3, I.FP32),     # binary32 rows: 14,322 units, 4 launches
    (900, 2048, 32, 2, 1, 0.0, I.BF16),      # 1,800 units: one launch
])
def test_sliced_combine_over_several_launches(T, H, E, K, A, mask, out_dtype):
    w = I.custom(f"split_comb{T}_{H}", 7500 + T, T, H, E, K, A, I.BF16, "uniform",
                 out_dtype=out_dtype, scales=False)
    _say(f"[sliced combine, launch limit {LIMIT}] {w}")
    case = I.make_case(w, mask_frac=mask)
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    dc = DeviceCase(case)
    dc.layout()
    got = dc.combine()
    torch.cuda.synchronize()
    if out_dtype == I.FP32:
        want = oracle.combine_f32(case.y, ref["dst_slot"], case.topk_weights)
        assert np.array_equal(to_host(got).view(np.uint32), want.view(np.uint32))
    else:
        want = oracle.combine(case.y, ref["dst_slot"], case.topk_weights)
        assert pins.bf16_ulp_distance(to_host(got, np.uint16), want).max() <= 1


@pytest.mark.parametrize("T,H,E,K,dtype,combine_fp32", [
    (200, 7168, 64, 8, I.BF16, False),   # 2,800 + 200 units: one launch, one unit per wave
    (400, 7168, 64, 8, I.BF16, False),   # 5,600 + 400 units: the looping kernel
    (400, 1024, 16, 2, I.FP8_E4M3, False),
    (333, 4096, 128, 6, I.BF16, True),   # binary32 combine rows: 16 slices
])
def test_non_expand_past_the_launch_limit(T, H, E, K, dtype, combine_fp32):
    w = I.custom(f"split_ne{T}_{H}", 7400 + T, T, H, E, K, 1, dtype, "uniform",
                 scales=dtype == I.FP8_E4M3)
    _run(w, mask=0.1, combine_fp32=combine_fp32)
