"""Host-side logic of bench.py (no GPU): the contract's refusals, the
algorithmic byte accounting, the counter scaling and the CPU baseline."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from combine_ep_layout_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# Closed forms per pass for every unmasked entry and received token (uniform
# routing never masks): layout T*K*4 (ids) + 8E + 4 (counts, offsets) +
# T*K*4 (slots) + T*(K+2)*4 (metadata) + 4 (num_recv); dispatch T*R + T*K*R +
# T*K*4; combine T*K*2H + T*2H + T*K*8, R = row bytes (+ 4 per 128-value
# scale block for fp8).
EXPECTED = {
    "tiny": (2184, 98_816, 99_328),
    "mori_default": (107_016, 132_153_344, 132_186_112),
    "decode_zipf": (15_368, 16_519_168, 16_523_264),
    "prefill_aligned": (428_040, 528_613_376, 528_744_448),
    "fp8_hot8": (854_024, 545_259_520, 1_057_488_896),
}


@pytest.mark.parametrize("name", list(EXPECTED))
def test_algorithmic_bytes_closed_forms(name):
    w = I.WORKLOADS[name]
    b = bench.algorithmic_bytes(w, w.T * w.K, w.T)
    assert (b["layout"], b["dispatch"], b["combine"]) == EXPECTED[name]


def test_non_expand_bytes_scale_with_received_tokens():
    w = I.WORKLOADS["prefill_aligned"]
    full = bench.algorithmic_bytes(w, w.T * w.K, w.T, "non-expand")
    half = bench.algorithmic_bytes(w, w.T * w.K // 2, w.T // 2, "non-expand")
    R = w.H * 2
    assert full["dispatch"] == 2 * w.T * R + w.T * (4 + 20 * w.K) + 4
    assert full["combine"] == w.T * (2 * w.H + 4) + w.T * (2 * w.H + 4 * w.K) + 4
    assert full["dispatch"] - half["dispatch"] == (w.T // 2) * (2 * R + 4 + 20 * w.K)


def test_fp4x2_combine_sees_two_values_per_byte():
    w = I.EXTRA_WORKLOADS["prefill_fp4x2"]
    row_in, scale_cols, H_out, elt_out = bench.geometry(w)
    assert H_out == 2 * w.H and scale_cols == 2 * w.H // 128 and row_in == w.H + 4 * scale_cols


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        wr.writeheader()
        for name, v in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Value": v})


def test_counter_scaling_uses_the_calibration_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    for rel in bench.KERNEL_SOURCES["expand"]:
        os.makedirs(os.path.dirname(tmp_path / rel), exist_ok=True)
        (tmp_path / rel).write_text(rel)
    gib_kib = (1 << 30) / 1024
    # calibration: FETCH reads half the true bytes, WRITE reads them exactly
    _counter_csv(tmp_path / "f.csv", [("at::native::neg_kernel", gib_kib / 2),
                                      ("ep::ep_combine_gather<0, 7168, 8, false, 256>", 1000.0),
                                      ("ep::ep_combine_gather<0, 7168, 8, false, 256>", 3000.0)])
    _counter_csv(tmp_path / "w.csv", [("at::native::neg_kernel", gib_kib),
                                      ("ep::ep_combine_gather<0, 7168, 8, false, 256>", 500.0),
                                      ("ep::ep_combine_gather<0, 7168, 8, false, 256>", 500.0)])
    out = bench.write_traffic("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    d = json.load(open(out))
    k = d["kernels"]["combine"]
    assert k["hbm_read_bytes"] == 2 * 2000 * 1024 and k["hbm_write_bytes"] == 500 * 1024
    assert bench.measured_traffic("wl", "combine") == 2 * 2000 * 1024 + 500 * 1024
    # a changed kernel source invalidates the stored counters
    (tmp_path / bench.KERNEL_SOURCES["expand"][0]).write_text("changed")
    assert bench.measured_traffic("wl", "combine") is None


def test_counters_without_calibration_are_refused(tmp_path):
    _counter_csv(tmp_path / "f.csv", [("ep::ep_combine_gather<0, 7168, 8, false, 256>", 1.0)])
    with pytest.raises(SystemExit):
        bench.write_traffic("wl", str(tmp_path / "f.csv"), str(tmp_path / "f.csv"))


@pytest.mark.parametrize("path", ["expand", "non-expand"])
def test_cpu_baseline_record(path):
    w = I.WORKLOADS["tiny"]
    case = I.make_case(w)
    if path == "non-expand":
        case.extra["y_ne"] = I.normal_bf16(w.seed, I.STREAM_Y, w.T, w.H)
    r = bench.cpu_baseline(case, budget_s=0.5, max_reps=2, path=path)
    assert r["kind"] == "oracle" and r["cores"] == bench.host_threads() and r["unit"] == "GB/s"
    assert r["value"] > 0 and "tiny" in r["sample"]
    assert r["single_thread"]["cores"] == 1 and r["single_thread"]["value"] > 0


@pytest.mark.parametrize("T,n", [(0, 4), (1, 8), (7, 3), (64, 64), (4096, 16), (1000, 7)])
def test_token_ranges_cover_every_token_once(T, n):
    """The all-threads CPU baseline splits the tokens into contiguous ranges: together
    they must cover every token exactly once, in order, with no empty range."""
    parts = bench._ranges(T, n)
    assert len(parts) <= n and all(b > a for a, b in parts)
    assert [t for a, b in parts for t in range(a, b)] == list(range(T))


def test_host_threads_respects_omp_cap(monkeypatch):
    monkeypatch.setenv("OMP_NUM_THREADS", "1")
    assert bench.host_threads() == 1
    monkeypatch.delenv("OMP_NUM_THREADS")
    assert bench.host_threads() >= 1


@pytest.mark.parametrize("T,K,E,one", [(128, 8, 256, True), (129, 8, 256, False), (64, 2, 16, True),
                                       (170, 6, 64, True), (171, 6, 64, False),
                                       (64, 8, 300, True), (65, 8, 300, False),
                                       (32, 8, 1024, True), (33, 8, 1024, False)])
def test_one_layout_tile_follows_the_tile_rule(T, K, E, one):
    """The step fuses layout and dispatch exactly when T*K fits one layout tile
    (floor(W / K) tokens, W by expert count, as the header states)."""
    assert bench.one_layout_tile(T, K, E) == one


def test_recorded_calls_replay_the_binding():
    """The per-kernel timing loop replays the C calls the binding would make: the
    recorder captures each function with its marshalled arguments and restores the
    library afterwards."""
    from combine_ep_layout_amd import binding as B
    L = B.lib()
    calls = bench.recorded_calls(B, lambda: [B.ep_set_workgroup_limit(None, 0) for _ in range(3)])
    assert B.lib() is L
    assert len(calls) == 3 and all(cfn is L.ep_set_workgroup_limit for cfn, _ in calls)
    assert all(cfn(*cargs) == 0 for cfn, cargs in calls)  # a cap of 0 on the null stream
