"""Benchmark: MoE expert-parallel layout + dispatch + combine on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input already resident in HBM: ep_layout (counts, aligned offsets, slots,
receive metadata), ep_dispatch (permute-copy into the expand buffer) and
ep_combine (weighted gather-reduce back to token order), all through the
C ABI on torch's current stream. Default workload: 4096 tokens, hidden 7168,
256 experts, top-8 uniform distinct routing, expert alignment 128, bf16.

Prints ONE JSON line. `value` is whole-step throughput: algorithmic HBM
bytes of the three passes per step divided by the wall-clock step time
(K steps bracketed by device synchronisation). Per-kernel times come from
HIP events recorded on the same stream around each call, on every Nth timed
step (--event-every, default 8: an event pair stalls the pipeline for a few
microseconds, so recording them on every step would slow the steps they
measure); the roofline
object reports the dominant kernel's algorithmic bytes over its mean event
duration against the MI355X HBM peak (8 TB/s). The CPU baseline times the
CPU oracle on the host (test infrastructure, never on the product path).
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "dispatch+combine effective HBM GB/s (% of peak) + tokens/s, 1 MI355X"
KERNEL_SOURCES = ["combine_ep_layout_amd/csrc/ep_dispatch.hip",
                  "combine_ep_layout_amd/csrc/ep_combine.hip",
                  "combine_ep_layout_amd/csrc/ep_layout.hip",
                  "combine_ep_layout_amd/csrc/ep_device.hpp"]


ELT_BYTES = {0: 2, 1: 4, 2: 1, 3: 1}  # bf16, fp32, fp8, fp4x2 (hidden counts bytes)
DTYPE_NAMES = {0: "bf16", 1: "f32", 2: "fp8_e4m3", 3: "fp4x2"}


def geometry(w):
    """Row bytes moved by dispatch (payload + scale row) and combine's row width and element size."""
    values = 2 * w.H if w.dtype == 3 else w.H
    scale_cols = values // 128 if (w.dtype in (2, 3) and w.scales) else 0
    row_in = w.H * ELT_BYTES[w.dtype] + 4 * scale_cols
    H_out = values  # combine sees one value per element
    return row_in, scale_cols, H_out, ELT_BYTES[w.out_dtype]


def algorithmic_bytes(w, n_valid: int, n_recv: int) -> dict:
    """Bytes each pass must move at minimum (padding rows are never touched)."""
    row_in, _, H_out, elt_out = geometry(w)
    L = w.T * w.K * 4 + 4 * w.E + 4 * (w.E + 1) + w.T * w.K * 4 + n_recv * (w.K + 2) * 4 + 4
    D = w.T * row_in + n_valid * row_in + w.T * w.K * 4
    C = n_valid * H_out * elt_out + w.T * H_out * elt_out + w.T * w.K * 8
    return {"layout": L, "dispatch": D, "combine": C}


def sources_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if current."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("sources_digest") != sources_digest():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


CALIBRATION_BYTES = 1 << 30  # fp32 elementwise negate: reads and writes this many bytes
KERNEL_TAGS = {"dispatch": "ep_dispatch_expand", "combine": "ep_combine_gather",
               "layout_histogram": "ep_layout_tile_histogram", "layout_assign": "ep_layout_tile_assign"}


def _counter_means(path: str) -> dict:
    """Mean counter value (KiB) per kernel-name tag from a rocprofv3 counter_collection CSV."""
    import csv
    sums, counts = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name", "")
            tag = None
            for k, t in KERNEL_TAGS.items():
                if t in name:
                    tag = k
            if tag is None and "neg_kernel" in name:
                tag = "calibration"
            if tag is None:
                continue
            v = float(r["Counter_Value"])
            sums[tag] = sums.get(tag, 0.0) + v
            counts[tag] = counts.get(tag, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def write_traffic(workload: str, fetch_csv: str, write_csv: str) -> str:
    """Turn FETCH_SIZE / WRITE_SIZE counter runs into HBM bytes per launch.

    Each counter is scaled by the factor that maps its reading for the
    calibration kernel (an fp32 negate of CALIBRATION_BYTES, which must read
    and write exactly that many bytes) to the true byte count.
    """
    fetch, write = _counter_means(fetch_csv), _counter_means(write_csv)
    if "calibration" not in fetch or "calibration" not in write:
        raise SystemExit("counter CSVs hold no calibration kernel: profile with --copy-calibration")
    f_scale = CALIBRATION_BYTES / (fetch["calibration"] * 1024.0)
    w_scale = CALIBRATION_BYTES / (write["calibration"] * 1024.0)
    kernels = {}
    for k in KERNEL_TAGS:
        if k in fetch and k in write:
            rd = fetch[k] * 1024.0 * f_scale
            wr = write[k] * 1024.0 * w_scale
            kernels[k] = {"fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                          "hbm_read_bytes": int(rd), "hbm_write_bytes": int(wr),
                          "hbm_bytes_per_launch": int(rd + wr)}
    out = {"workload": workload, "sources_digest": sources_digest(),
           "calibration": {"kernel": "torch.neg fp32, 1 GiB in, 1 GiB out",
                           "fetch_kib": round(fetch["calibration"], 1),
                           "write_kib": round(write["calibration"], 1),
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "kernels": kernels}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return path


def cpu_baseline(case, budget_s: float = 10.0, max_reps: int = 5):
    """Time the CPU oracle (as it stands) on the same workload on the host."""
    import oracle

    w = case.w
    rowb = case.x.view(np.uint8).reshape(w.T, -1).shape[1]
    expand = np.zeros((w.cap, rowb), np.uint8)
    expand_s = (np.zeros((w.cap, case.x_scales.shape[1] * 4), np.uint8)
                if case.x_scales is not None else None)
    times = []
    t_start = time.perf_counter()
    while len(times) < max_reps and (len(times) < 2 or time.perf_counter() - t_start < budget_s):
        t0 = time.perf_counter()
        lay = oracle.layout(case.topk_idx, w.E, w.A)
        oracle.dispatch(case.x, lay["dst_slot"], w.cap, x_scales=case.x_scales,
                        expand_x=expand, expand_scales=expand_s)
        if w.out_dtype == 1:
            oracle.combine_f32(case.y, lay["dst_slot"], case.topk_weights)
        else:
            oracle.combine(case.y, lay["dst_slot"], case.topk_weights)
        times.append(time.perf_counter() - t0)
    n_valid = int((lay["dst_slot"] >= 0).sum())
    b = algorithmic_bytes(w, n_valid, lay["num_recv"])
    sec = float(np.median(times))
    return {"value": round(sum(b.values()) / sec / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "seconds_per_step": round(sec, 3),
            "sample": f"the full {w.name} workload (layout + dispatch + combine), "
                      f"{len(times)} single-threaded runs, median"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_aligned")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=8,
                    help="record per-kernel HIP events on every Nth timed step (each event "
                         "pair costs a few microseconds of pipeline bubble)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB fp32 negate first (a plain streaming kernel of known size "
                         "for scaling hardware byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 FETCH_SIZE and "
                         "WRITE_SIZE counter CSVs, then exit")
    args = ap.parse_args()
    if args.traffic_from:
        print(write_traffic(args.workload, *args.traffic_from))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every expert is local, a world of one); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from combine_ep_layout_amd import binding as B
    from combine_ep_layout_amd import inputs as I

    B.lib()  # fail loudly if the HIP library is not built
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = {**I.WORKLOADS, **I.EXTRA_WORKLOADS}[args.workload]
    print(f"# workload {w.name}: T={w.T} H={w.H} E={w.E} K={w.K} A={w.A} dtype={w.dtype} "
          f"cap={w.cap}", file=sys.stderr, flush=True)
    case = I.make_case(w)

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    idx, wts, x, y = up(case.topk_idx), up(case.topk_weights), up(case.x), up(case.y)
    xs = up(case.x_scales) if case.x_scales is not None else None
    rowb = case.x.view(np.uint8).reshape(w.T, -1).shape[1]
    _, scale_cols, H_out, _ = geometry(w)
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
    dst = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    meta = torch.empty((w.T, w.K + 2), dtype=torch.int32, device=dev)
    nrecv = torch.empty(1, dtype=torch.int32, device=dev)
    wsb = B.ep_layout_workspace_bytes(w.T, w.K, w.E)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    expand = torch.zeros((w.cap, rowb), dtype=torch.uint8, device=dev)
    expand_s = (torch.zeros((w.cap, scale_cols), dtype=torch.float32, device=dev)
                if xs is not None else None)
    out = torch.empty((w.T, H_out), dtype=torch.float32 if w.out_dtype == 1 else torch.int16,
                      device=dev)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        a = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        B.ep_layout(idx, w.T, w.K, w.E, w.A, w.cap, counts, offsets, dst, meta, nrecv, ws, wsb, stream)
        if ev is not None:
            ev[1].record(stream)
        B.ep_dispatch(x, xs, None, dst, w.T, w.H, w.K, w.dtype, w.cap, expand, expand_s, None, stream)
        if ev is not None:
            ev[2].record(stream)
        B.ep_combine(y, wts, None, dst, w.T, H_out, w.K, w.out_dtype, w.cap, out, stream)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    every = max(1, args.event_every)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(0, args.steps, every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i // every] if i % every == 0 else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    us = {"layout": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e3,
          "dispatch": float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e3,
          "combine": float(np.mean([e[2].elapsed_time(e[3]) for e in evs])) * 1e3}

    # Validate the timed path against the oracle: layout in full, dispatch and combine sampled.
    import oracle
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    got_dst = dst.cpu().numpy()
    ok = (np.array_equal(got_dst, ref["dst_slot"]) and np.array_equal(offsets.cpu().numpy(), ref["offsets"])
          and np.array_equal(counts.cpu().numpy(), ref["counts"]) and int(nrecv.item()) == ref["num_recv"])
    sample = np.random.default_rng(0).choice(w.T, size=min(w.T, 256), replace=False)
    xb = case.x.view(np.uint8).reshape(w.T, -1)
    rows = ref["dst_slot"][sample]
    got_rows = expand[torch.from_numpy(rows.ravel().astype(np.int64)).to(dev)].cpu().numpy()
    ok = ok and np.array_equal(got_rows, np.repeat(xb[sample], w.K, axis=0))
    if w.out_dtype == 1:
        ref_out = oracle.combine_f32(case.y, ref["dst_slot"][sample], case.topk_weights[sample])
        ok = ok and np.array_equal(out.cpu().numpy()[sample].view(np.uint32), ref_out.view(np.uint32))
    else:
        ref_out = oracle.combine(case.y, ref["dst_slot"][sample], case.topk_weights[sample])
        got_out = out.cpu().numpy().view(np.uint16)[sample]
        ordered = lambda b: np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + b)  # noqa: E731
        ok = ok and np.abs(ordered(got_out.astype(np.int32))
                           - ordered(ref_out.astype(np.int32))).max() <= 1
    if not ok:
        print("bench: GPU results do not match the oracle; refusing to report", file=sys.stderr)
        sys.exit(1)

    n_valid = int((ref["dst_slot"] >= 0).sum())
    nb = algorithmic_bytes(w, n_valid, ref["num_recv"])
    total_bytes = sum(nb.values())
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    dc_us = us["dispatch"] + us["combine"]
    dc_gbps = (nb["dispatch"] + nb["combine"]) / (dc_us * 1e-6) / 1e9
    dom = max(("dispatch", "combine"), key=lambda k: us[k])
    achieved = nb[dom] / (us[dom] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(w.name, dom),
                "algorithmic_bytes_per_launch": nb[dom], "avg_launch_us": round(us[dom], 2)}
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[w.dtype] if w.out_dtype == 0 else
                 f"{DTYPE_NAMES[w.dtype]}->{DTYPE_NAMES[w.out_dtype]}",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E, "topk": w.K,
                   "expert_alignment": w.A, "capacity_rows": w.cap, "routing": w.routing,
                   "dispatch_dtype": DTYPE_NAMES[w.dtype], "combine_dtype": DTYPE_NAMES[w.out_dtype],
                   "parallelism": "one GPU, all experts local"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(w.T / (ms_per_step * 1e-3), 1),
        "dispatch_combine_GBps": round(dc_gbps, 1),
        "dispatch_combine_pct_of_peak": round(100 * dc_gbps / HBM_PEAK_GBPS, 2),
        "dispatch_combine_tokens_per_s": round(w.T / (dc_us * 1e-6), 1),
        "kernel_us": {k: round(v, 2) for k, v in us.items()},
        "algorithmic_bytes": nb,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
