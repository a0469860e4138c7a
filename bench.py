"""Benchmark: MoE expert-parallel layout + dispatch + combine on one MI355X.

One step is one pass of the whole hot path over one batch of synthetic
input already resident in HBM: ep_layout (counts, aligned offsets, slots,
receive metadata), ep_dispatch (permute-copy into the expand buffer) and
ep_combine (weighted gather-reduce back to token order), all through the
C ABI on torch's current stream. Default workload: 4096 tokens, hidden 7168,
256 experts, top-8 uniform distinct routing, expert alignment 128, bf16.

--path non-expand times the other layout mode instead: ep_layout,
ep_dispatch_compact (one row per received token, with its expert ids and
router weights) and ep_combine_compact (rows back to token order).
A batch that fits one layout tile (a decode step) calls ep_layout_dispatch
(ep_layout_dispatch_compact) instead of the first two calls: one launch;
--no-fused keeps them apart, --one-call uses the fused call at every batch
size (on the expand path with ep_layout_dispatch_workspace_bytes, so that
large batches walk the plan it keeps in the workspace). On the expand path
every batch of more than one layout tile asks the layout for the dispatch
plan and dispatches by it (--no-plan: token-major).
--read-ahead hands x to ep_layout as its read-ahead region, so that x is in
the last-level cache when dispatch starts.
Each run times two cache modes (--cache both, the default; --cache warm or
--cache cold, or --cold, times one). Warm: steps back to back on one buffer
set, so x, read by the step before, is still in the 256 MB last-level cache
(MALL), as when the router GEMM has just touched it. Cold: the step rotates
several complete sets of buffers (expert outputs, expand / receive buffers,
out), enough that at least 512 MB of other traffic separates two uses of a
set, and separately enough copies of x (with its scale rows) that at least
512 MB of other x reads separate two uses of a copy. Only ordinary loads fill
the MALL; the rest of the step's traffic is non-temporal and leaves it alone,
so rotating x among its own copies is what makes each step find x in HBM.
Nothing but steps runs in the timed loop. Every run also times torch's copy_
of 1 GiB (16-byte vector loads and stores) and reports the path as a
fraction of that copy.
--graph N captures N consecutive steps in one hipGraph and times its
replays for `value` (per-kernel times still come from the eager pass): the
launch cost a caller pays when it captures several layers together.
--workgroups L runs the step on a stream capped at L workgroups (the
CU-limited mode); --overlap-gemm additionally times a bf16 GEMM on a second
stream alone and interleaved with the steps, and reports how much of the
shorter of the two the overlap hides.

Prints ONE JSON line: the first mode's figures at the top level, the other
mode's in an object named after it ("cold" by default). `value` is
whole-step throughput: algorithmic HBM bytes of the three passes per step
divided by the wall-clock step time (K steps bracketed by device
synchronisation, no events inside; the steps' C calls are marshalled
beforehand and made directly, as a native caller would make them, so the
Python binding's per-call work does not set the pace of small steps).
Warm-up: about 25 ms (at most 512 steps) of untimed steps queued back to
back, then the W warm-up steps, then the timed steps, each after a
synchronisation. After an idle spell this GPU runs a memory-bound load
about 10% slower from about 2 ms to about 10 ms into it; a short run that
started from idle would time that dip, not the path (warmup_steps_run
counts every untimed step). Per-kernel times come right after the timed
loop: each pass is launched a few times untimed and
then --event-steps times (default 50, at least 20) back to back with the
step's buffer rotation, the timed launches between two HIP events, after
the same untimed load and queued behind a GPU spin of under 1 ms that holds
the stream until the host has issued every call; kernel_us is the mean per
launch (an event drains the pipeline, about 3 us, so events around each
single launch would read several microseconds above the kernel's own
duration as rocprofv3 reports it). The roofline object reports the dominant
kernel's algorithmic bytes over that mean against the MI355X HBM peak
(8 TB/s). The CPU baseline times the CPU oracle on the host, on one thread
and on all host threads (test infrastructure, never on the product path).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
N_PRE_LAUNCHES = 5  # untimed launches of a pass before its per-kernel events
GATE_CYCLES_PER_LAUNCH = 35_000  # GPU spin ahead of the timed launches, per launch queued
LOAD_MS = 25.0  # untimed full steps, back to back, before each timed region
LOAD_CHUNK_STEPS = 8  # steps per chunk of that load (one chunk is timed to size it)
LOAD_MAX_STEPS = 512  # bound on the steps queued for that load
METRIC = "dispatch+combine effective HBM GB/s (% of peak) + tokens/s, 1 MI355X"
KERNEL_SOURCES = {  # the sources whose kernels each path's traffic counters measured
    "expand": ["combine_ep_layout_amd/csrc/ep_dispatch.hip",
               "combine_ep_layout_amd/csrc/ep_combine.hip",
               "combine_ep_layout_amd/csrc/ep_layout.hip",
               "combine_ep_layout_amd/csrc/ep_device.hpp"],
    "non-expand": ["combine_ep_layout_amd/csrc/ep_compact.hip",
                   "combine_ep_layout_amd/csrc/ep_layout.hip",
                   "combine_ep_layout_amd/csrc/ep_device.hpp"],
}


ELT_BYTES = {0: 2, 1: 4, 2: 1, 3: 1}  # bf16, fp32, fp8, fp4x2 (hidden counts bytes)
DTYPE_NAMES = {0: "bf16", 1: "f32", 2: "fp8_e4m3", 3: "fp4x2"}


def geometry(w):
    """Row bytes moved by dispatch (payload + scale row) and combine's row width and element size."""
    values = 2 * w.H if w.dtype == 3 else w.H
    scale_cols = values // 128 if (w.dtype in (2, 3) and w.scales) else 0
    row_in = w.H * ELT_BYTES[w.dtype] + 4 * scale_cols
    H_out = values  # combine sees one value per element
    return row_in, scale_cols, H_out, ELT_BYTES[w.out_dtype]


def algorithmic_bytes(w, n_valid: int, n_recv: int, path: str = "expand") -> dict:
    """Bytes each pass must move at minimum (padding rows are never touched).

    expand: dispatch reads each token row once and writes it per unmasked
    entry; combine reads each entry's row and writes each token's row.
    non-expand: dispatch reads and writes one row per received token plus its
    K ids (topk_idx and dst_slot read, recv_topk_idx written) and K weights
    (read and written) and its metadata token column; combine reads one row
    per received token and its metadata column, reads every token's K slots
    (to find tokens that received nothing) and writes every token's row.
    """
    row_in, _, H_out, elt_out = geometry(w)
    L = w.T * w.K * 4 + 4 * w.E + 4 * (w.E + 1) + w.T * w.K * 4 + n_recv * (w.K + 2) * 4 + 4
    if path == "non-expand":
        D = 2 * n_recv * row_in + n_recv * (4 + 5 * 4 * w.K) + 4
        C = n_recv * (H_out * elt_out + 4) + w.T * (H_out * elt_out + 4 * w.K) + 4
        return {"layout": L, "dispatch": D, "combine": C}
    D = w.T * row_in + n_valid * row_in + w.T * w.K * 4
    C = n_valid * H_out * elt_out + w.T * H_out * elt_out + w.T * w.K * 8
    return {"layout": L, "dispatch": D, "combine": C}


def _code_only(text: str) -> str:
    """C++ source without comments and whitespace: edits to either leave the kernels unchanged."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def sources_digest(path_mode: str = "expand") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[path_mode]:
        with open(os.path.join(ROOT, rel)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if current."""
    path_mode = "non-expand" if kernel.endswith("_compact") else "expand"
    suffix = "_non_expand" if path_mode == "non-expand" else ""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}{suffix}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("sources_digest") != sources_digest(path_mode):
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def one_layout_tile(T: int, K: int, E: int) -> bool:
    """Whether ep_layout_dispatch runs as one launch: T*K fits one layout tile
    of floor(W / K) tokens, W = 1024, 512 or 256 for E up to 256, 512, 1024."""
    W = 1024 if E <= 256 else (512 if E <= 512 else 256)
    return T <= W // K


CALIBRATION_BYTES = 1 << 30  # fp32 elementwise negate: reads and writes this many bytes
# Kernel-name fragments per pass: each pass launches one of its kernels, chosen by shape and cap
# (a one-tile batch's layout + dispatch kernel counts as dispatch, as its time does).
KERNEL_TAGS = {"dispatch": ("ep_dispatch_expand", "ep_dispatch_grouped", "ep_dispatch_fanout",
                            "ep_layout_dispatch_tile"),
               "combine": ("ep_combine_stream", "ep_combine_gather"),
               "dispatch_compact": ("ep_dispatch_compact_rows", "ep_layout_dispatch_compact_tile"),
               "combine_compact": ("ep_combine_compact_rows",),
               "layout_histogram": ("ep_layout_tile_histogram",),
               "layout_assign": ("ep_layout_tile_assign",)}


def _counter_means(path: str) -> dict:
    """Mean counter value (KiB) per kernel-name tag from a rocprofv3 counter_collection CSV."""
    import csv
    sums, counts = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = r.get("Kernel_Name", "")
            tag = None
            for k, frags in KERNEL_TAGS.items():
                if any(f in name for f in frags):
                    tag = k
            if tag is None and "neg_kernel" in name:
                tag = "calibration"
            if tag is None:
                continue
            v = float(r["Counter_Value"])
            sums[tag] = sums.get(tag, 0.0) + v
            counts[tag] = counts.get(tag, 0) + 1
    return {k: sums[k] / counts[k] for k in sums}


def write_traffic(workload: str, fetch_csv: str, write_csv: str, path_mode: str = "expand") -> str:
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
    out = {"workload": workload, "path": path_mode, "sources_digest": sources_digest(path_mode),
           "calibration": {"kernel": "torch.neg fp32, 1 GiB in, 1 GiB out",
                           "fetch_kib": round(fetch["calibration"], 1),
                           "write_kib": round(write["calibration"], 1),
                           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)},
           "kernels": kernels}
    suffix = "_non_expand" if path_mode == "non-expand" else ""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}{suffix}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    return path


def host_threads() -> int:
    """Threads the CPU baseline may use: the CPUs this process may run on, capped
    by OMP_NUM_THREADS when the host sets it (a share of a larger machine)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _ranges(T: int, n: int):
    """n contiguous token ranges covering [0, T)."""
    cuts = [T * i // n for i in range(n + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(n) if cuts[i + 1] > cuts[i]]


def cpu_baseline(case, budget_s: float = 8.0, max_reps: int = 100_000, path: str = "expand"):
    """Time the CPU oracle (as it stands) on the same workload on the host.

    Two figures, each whole steps repeated until budget_s seconds (at least two
    runs), median: one host thread; and all host threads, where the layout
    stays one sequential call and dispatch and combine are split over
    contiguous token ranges, one per thread, each thread calling the same
    oracle functions on its range (ctypes releases the interpreter lock
    during the C calls). Per-token arithmetic is unchanged, so the results
    are the same; only the wall time differs.
    """
    import concurrent.futures as cf

    import oracle

    w = case.w
    n_threads = host_threads()
    pool = cf.ThreadPoolExecutor(max_workers=n_threads) if n_threads > 1 else None

    def split(fn, parts):
        if pool is None or len(parts) == 1:
            for a, b in parts:
                fn(a, b)
        else:
            list(pool.map(lambda r: fn(*r), parts))

    if path == "non-expand":
        y = case.extra["y_ne"]
        combine_rows = oracle.combine_compact_f32 if w.out_dtype == 1 else oracle.combine_compact

        def one_step(parts):
            lay = oracle.layout(case.topk_idx, w.E, w.A)
            meta, n = lay["recv_src_metadata"], lay["num_recv"]
            def disp(a, b):  # received rows are in token order: a token range is a row range
                i0, i1 = np.searchsorted(meta[:, 0], [a, b])
                oracle.dispatch_compact(case.x, case.topk_idx, lay["dst_slot"], meta[i0:i1],
                                        i1 - i0, case.x_scales, case.topk_weights)

            def comb(a, b):  # the range's received rows, token column taken relative to a
                i0, i1 = np.searchsorted(meta[:, 0], [a, b])
                m = meta[i0:i1].copy()
                m[:, 0] -= a
                combine_rows(y[i0:i1], lay["dst_slot"][a:b], m, i1 - i0)

            split(disp, parts)
            split(comb, parts)
            return lay
        label = "non-expand (layout + dispatch_compact + combine_compact)"
    else:
        rowb = case.x.view(np.uint8).reshape(w.T, -1).shape[1]
        expand = np.zeros((w.cap, rowb), np.uint8)
        expand_s = (np.zeros((w.cap, case.x_scales.shape[1] * 4), np.uint8)
                    if case.x_scales is not None else None)

        def one_step(parts):
            lay = oracle.layout(case.topk_idx, w.E, w.A)
            dst = lay["dst_slot"]

            def disp(a, b):
                oracle.dispatch(case.x[a:b], dst[a:b], w.cap,
                                x_scales=None if case.x_scales is None else case.x_scales[a:b],
                                expand_x=expand, expand_scales=expand_s)

            def comb(a, b):
                if w.out_dtype == 1:
                    oracle.combine_f32(case.y, dst[a:b], case.topk_weights[a:b])
                else:
                    oracle.combine(case.y, dst[a:b], case.topk_weights[a:b])

            split(disp, parts)
            split(comb, parts)
            return lay
        label = "(layout + dispatch + combine)"

    def timed(parts):
        times = []
        t_start = time.perf_counter()
        lay = None
        while len(times) < max_reps and (len(times) < 2 or time.perf_counter() - t_start < budget_s):
            t0 = time.perf_counter()
            lay = one_step(parts)
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(times), sum(times), lay

    sec1, n1, tot1, lay = timed([(0, w.T)])
    secn, nn, totn, _ = timed(_ranges(w.T, n_threads)) if n_threads > 1 else (sec1, n1, tot1, lay)
    if pool is not None:
        pool.shutdown()
    n_valid = int((lay["dst_slot"] >= 0).sum())
    b = sum(algorithmic_bytes(w, n_valid, lay["num_recv"], path).values())
    return {"value": round(b / secn / 1e9, 3), "unit": "GB/s", "cores": n_threads,
            "kind": "oracle", "seconds_per_step": round(secn, 4),
            "single_thread": {"value": round(b / sec1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "seconds_per_step": round(sec1, 4)},
            "host_cpus": os.cpu_count(),
            "sample": f"the full {w.name} workload {label}: {n1} single-threaded steps in "
                      f"{tot1:.1f} s and {nn} steps on {n_threads} threads in {totn:.1f} s, "
                      f"medians; the layout runs on one thread, dispatch and combine are "
                      f"split over {n_threads} contiguous token ranges"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill_aligned")
    ap.add_argument("--path", choices=("expand", "non-expand"), default="expand",
                    help="expand: one row per (token, expert) (the default, headline path); "
                         "non-expand: one row per received token")
    ap.add_argument("--no-plan", action="store_true",
                    help="expand path: never ask ep_layout for the dispatch plan (by default every "
                         "batch of more than one layout tile dispatches by it)")
    ap.add_argument("--read-ahead", action="store_true",
                    help="hand x to ep_layout as its read-ahead region: the layout's launches "
                         "pull x into the last-level cache for dispatch (helps a cold x, costs a "
                         "few microseconds when x is cached)")
    ap.add_argument("--one-call", action="store_true",
                    help="run layout and dispatch through ep_layout_dispatch "
                         "(ep_layout_dispatch_compact) at every batch size, not only for one-tile "
                         "batches (with the plan-sized workspace on the expand path)")
    ap.add_argument("--no-fused", action="store_true",
                    help="call ep_layout and ep_dispatch (ep_dispatch_compact) separately even "
                         "when the batch fits one layout tile (by default ep_layout_dispatch "
                         "(ep_layout_dispatch_compact) is used then)")
    ap.add_argument("--cache", choices=("both", "warm", "cold"), default="both",
                    help="warm: steps back to back on one buffer set; cold: rotate buffer sets "
                         "and copies of x so that no step finds its rows in the last-level "
                         "cache; both (default): the warm line with a `cold` object beside it")
    ap.add_argument("--cold", action="store_true", help="same as --cache cold")
    ap.add_argument("--workgroups", type=int, default=0,
                    help="cap every kernel of the step at this many workgroups (0: no cap)")
    ap.add_argument("--graph", type=int, default=0, metavar="N",
                    help="time replays of a hipGraph holding N steps (0: eager launches)")
    ap.add_argument("--overlap-gemm", action="store_true",
                    help="also time a bf16 GEMM on a second stream, alone and overlapped")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-steps", type=int, default=50,
                    help="launches of each pass timed back to back between two HIP events after "
                         "the timed loop, for the per-kernel times (at least 20)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB fp32 negate first (a plain streaming kernel of known size "
                         "for scaling hardware byte counters)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 FETCH_SIZE and "
                         "WRITE_SIZE counter CSVs, then exit")
    args = ap.parse_args()
    if args.traffic_from:
        print(write_traffic(args.workload, *args.traffic_from, path_mode=args.path))
        return
    if args.graph and args.workgroups:
        raise SystemExit("--graph and --workgroups do not combine: a capture runs on its own stream")
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
    case = I.make_case(w, with_y=args.path == "expand")
    non_expand = args.path == "non-expand"

    def up(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    _, scale_cols, H_out, _ = geometry(w)
    if non_expand:
        # the expert side's reduced output: one row per received token, of combine's type
        case.extra["y_ne"] = (I.normal_bf16(w.seed, I.STREAM_Y, w.T, H_out) if w.out_dtype == 0
                              else I.normal_f32(w.seed, I.STREAM_Y, w.T, H_out))
        case.y = case.extra["y_ne"]
    idx, wts = up(case.topk_idx), up(case.topk_weights)
    rowb = case.x.view(np.uint8).reshape(w.T, -1).shape[1]
    counts = torch.empty(w.E, dtype=torch.int32, device=dev)
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
    dst = torch.empty((w.T, w.K), dtype=torch.int32, device=dev)
    meta = torch.empty((w.T, w.K + 2), dtype=torch.int32, device=dev)
    nrecv = torch.empty(1, dtype=torch.int32, device=dev)
    one_tile = one_layout_tile(w.T, w.K, w.E)
    fused = not args.no_fused and (one_tile or args.one_call)
    wsb = (B.ep_layout_dispatch_workspace_bytes(w.T, w.K, w.E)
           if fused and not non_expand and not args.no_plan
           else B.ep_layout_workspace_bytes(w.T, w.K, w.E))
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    rows_out = w.T if non_expand else w.cap
    # The capped fan-out dispatch ignores a plan, so a capped step does not ask for one.
    use_plan = not non_expand and not args.no_plan and not fused and not args.workgroups
    plan = torch.empty((w.T * w.K, 2), dtype=torch.int32, device=dev) if use_plan else None

    def x_set():
        """One copy of the tokens' rows and scale rows."""
        return {"x": up(case.x),
                "xs": up(case.x_scales) if case.x_scales is not None else None}

    def buffer_set():
        """The other rows one step reads and writes (the small layout arrays are shared)."""
        return {
            "y": up(case.y),
            "expand": torch.zeros((rows_out, rowb), dtype=torch.uint8, device=dev),
            "expand_s": (torch.zeros((rows_out, scale_cols), dtype=torch.float32, device=dev)
                         if case.x_scales is not None else None),
            "recv_i": torch.empty((w.T, w.K), dtype=torch.int32, device=dev) if non_expand else None,
            "recv_w": torch.empty((w.T, w.K), dtype=torch.float32, device=dev) if non_expand else None,
            "out": torch.empty((w.T, H_out), dtype=torch.float32 if w.out_dtype == 1 else torch.int16,
                               device=dev),
        }

    step_bytes = sum(algorithmic_bytes(w, w.T * w.K, w.T, args.path).values())
    x_bytes = case.x.nbytes + (case.x_scales.nbytes if case.x_scales is not None else 0)
    stream = torch.cuda.current_stream()
    if args.workgroups > 0:
        stream = torch.cuda.Stream()  # default priority
        B.ep_set_workgroup_limit(stream, args.workgroups)
        print(f"# workgroup cap {B.ep_get_workgroup_limit(stream)}", file=sys.stderr, flush=True)
    copy_gbps = copy_reference(torch, dev)
    if args.copy_calibration:
        a = torch.ones(CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b

    import oracle
    ref = oracle.layout(case.topk_idx, w.E, w.A)
    sample = np.random.default_rng(0).choice(w.T, size=min(w.T, 256), replace=False)
    xb = case.x.view(np.uint8).reshape(w.T, -1)

    def run_mode(cold: bool, first: bool) -> dict:
        """Warm-up, the K timed steps, then the instrumented pass; validates the results."""
        nsets = nx = 1
        if cold:  # at least 512 MB of other traffic between two uses of a set or an x copy
            nsets = min(32, max(2, -(-(512 << 20) // step_bytes) + 1))
            nx = min(1024, max(2, -(-(512 << 20) // x_bytes) + 1))
        sets = [buffer_set() for _ in range(nsets)]
        x_sets = [x_set() for _ in range(nx)]

        def run_layout(i, stream=stream):
            S, X = sets[i % nsets], x_sets[i % nx]
            if fused and non_expand:  # one launch; its time is reported as dispatch's
                B.ep_layout_dispatch_compact(idx, w.T, w.K, w.E, w.A, w.cap, counts, offsets, dst,
                                             meta, nrecv, ws, wsb, X["x"], X["xs"], wts, w.H,
                                             w.dtype, S["expand"], S["expand_s"], S["recv_i"],
                                             S["recv_w"], stream)
            elif fused:
                B.ep_layout_dispatch(idx, w.T, w.K, w.E, w.A, w.cap, counts, offsets, dst, meta,
                                     nrecv, ws, wsb, X["x"], X["xs"], None, w.H, w.dtype,
                                     S["expand"], S["expand_s"], None, stream)
            else:
                B.ep_layout(idx, w.T, w.K, w.E, w.A, w.cap, counts, offsets, dst, meta, nrecv, ws,
                            wsb, stream, dispatch_plan=plan,
                            prefetch=X["x"] if args.read_ahead else None)

        def run_dispatch(i, stream=stream):
            S, X = sets[i % nsets], x_sets[i % nx]
            if non_expand and not fused:
                B.ep_dispatch_compact(X["x"], X["xs"], idx, wts, dst, meta, nrecv, w.T, w.H, w.K,
                                      w.dtype, S["expand"], S["expand_s"], S["recv_i"],
                                      S["recv_w"], stream)
            elif not non_expand and not fused:
                B.ep_dispatch(X["x"], X["xs"], None, dst, w.T, w.H, w.K, w.dtype, w.cap,
                              S["expand"], S["expand_s"], None, stream, dispatch_plan=plan)

        def run_combine(i, stream=stream):
            S = sets[i % nsets]
            if non_expand:
                B.ep_combine_compact(S["y"], None, dst, meta, nrecv, w.T, H_out, w.K, w.out_dtype,
                                     S["out"], stream)
            else:
                B.ep_combine(S["y"], wts, None, dst, w.T, H_out, w.K, w.out_dtype, w.cap, S["out"],
                             stream)

        def step(i, stream=stream):
            run_layout(i, stream)
            run_dispatch(i, stream)
            run_combine(i, stream)

        def issue(calls) -> int:
            failed = 0
            for cfn, cargs in calls:
                failed |= cfn(*cargs)
            return failed

        torch.cuda.synchronize()  # inputs were written on the default stream
        # Every call is marshalled before any of them runs (the library's C
        # functions with their arguments, made directly as a native caller
        # would: the binding's per-call Python work, about 5 us, would
        # otherwise set the pace of small steps), so no host work leaves the
        # GPU idle between the warm-up and the timed steps.
        n_warm = max(args.warmup, nsets, nx)
        warm_calls = recorded_calls(B, lambda: [step(i) for i in range(n_warm)])
        timed_calls = recorded_calls(B, lambda: [step(i) for i in range(args.steps)])
        load_calls = recorded_calls(B, lambda: [step(i) for i in range(LOAD_CHUNK_STEPS)])

        def load() -> int:
            """About LOAD_MS of untimed full steps, queued back to back; returns how many.

            After an idle spell this GPU runs a memory-bound load at full speed
            for about 2 ms, then about 10% slower for about 8 ms before it
            settles (dispatch at prefill: 75, then up to 84-90, then 75 us), and
            a load broken by a synchronisation every few steps does not reach
            the settled state (20 prefill steps timed after 25 ms of such a load
            read 177 against 168 us). So a chunk is timed to size the load (the
            second of two: a process's first steps also pay for first touches
            of their buffers), and the rest is queued without waiting; the
            caller's next work follows it in the queue. At most LOAD_MAX_STEPS
            steps are queued: after a burst of some thousands of short launches
            (decode steps, whose chunk is mostly host time) the next launches
            took about 200 us longer in all, and short steps draw too little
            power for the dip to matter.
            """
            for _ in range(2):
                t0 = time.perf_counter()
                if issue(load_calls):
                    raise SystemExit(f"bench: an untimed step failed: {B.ep_last_error()}")
                torch.cuda.synchronize()
                chunk_ms = (time.perf_counter() - t0) * 1e3
            chunks = min(LOAD_MAX_STEPS // LOAD_CHUNK_STEPS,
                         max(1, int(LOAD_MS / max(chunk_ms, 1e-3))))
            for _ in range(chunks):
                if issue(load_calls):
                    raise SystemExit(f"bench: an untimed step failed: {B.ep_last_error()}")
            return (chunks + 2) * LOAD_CHUNK_STEPS

        def drain():
            """torch.cuda.synchronize(), after polling an event recorded behind
            the queued work, so the host thread stays awake through a long
            wait: a host-bound step (decode) issued right after a blocking wait
            of several ms ran slower for a while (20 decode steps: 17.5 against
            12.8 us each)."""
            ev = torch.cuda.Event()
            ev.record(stream)
            while not ev.query():
                pass
            torch.cuda.synchronize()

        n_load = load()
        drain()
        if issue(warm_calls):
            raise SystemExit(f"bench: a warm-up step failed: {B.ep_last_error()}")
        drain()
        t0 = time.perf_counter()
        failed = issue(timed_calls)  # the timed region: steps only, no events
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        if failed:
            raise SystemExit(f"bench: a timed call failed: {B.ep_last_error()}")
        # Per-kernel times: right after the timed loop, each pass is launched
        # n_ev times back to back on the same stream, with the step's buffer
        # rotation, between two HIP events (an event drains the pipeline, about
        # 3 us each, so events around single launches would read several
        # microseconds above the kernel's own duration); the mean per launch
        # is the kernel's average duration. Before each series the GPU is
        # loaded with full steps (load(): no post-idle dip inside the series),
        # then a bounded GPU spin (under 1 ms) holds the stream while the host
        # issues every call, so the launches run back to back even where a
        # call takes as long on the host as its launches on the GPU (the
        # layout's, decode's). A few untimed launches of the same pass precede
        # the first event, on buffer sets the timed loop has just used (so a
        # cold pass stays cold).
        n_ev = max(20, args.event_steps)
        n_pre = min(N_PRE_LAUNCHES, args.steps)
        us = {}
        for name, fn in (("layout", run_layout), ("dispatch", run_dispatch),
                         ("combine", run_combine)):
            pre = recorded_calls(B, lambda: [fn(args.steps - n_pre + j) for j in range(n_pre)])
            calls = recorded_calls(B, lambda: [fn(args.steps + j) for j in range(n_ev)])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            load()
            with torch.cuda.stream(stream):
                torch.cuda._sleep(GATE_CYCLES_PER_LAUNCH * (n_ev + n_pre))
            failed = issue(pre)
            e0.record(stream)
            failed |= issue(calls)
            e1.record(stream)
            torch.cuda.synchronize()
            if failed:
                raise SystemExit(f"bench: {name} failed: {B.ep_last_error()}")
            us[name] = e0.elapsed_time(e1) * 1e3 / n_ev
        if fused:  # layout ran inside the dispatch launch
            us = {"layout": 0.0, "dispatch": us["layout"], "combine": us["combine"]}
        launch = "eager"
        if first and args.graph > 0:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(args.graph):
                    step(i, stream=torch.cuda.current_stream())
            for _ in range(3):
                g.replay()
            reps = max(1, args.steps // args.graph)
            load()
            drain()
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            ms_per_step = (time.perf_counter() - t0) * 1e3 / (reps * args.graph)
            launch = f"hipGraph of {args.graph} steps, {reps} replays"
        overlap = (overlap_gemm(torch, dev, lambda: step(0), ms_per_step, args.steps)
                   if first and args.overlap_gemm else None)
        torch.cuda.synchronize()
        # Validate this mode's results against the oracle: layout in full,
        # dispatch and combine on sampled tokens (every set holds the same rows).
        last = sets[(args.steps + n_ev - 1) % nsets]
        ok = (np.array_equal(dst.cpu().numpy(), ref["dst_slot"])
              and np.array_equal(offsets.cpu().numpy(), ref["offsets"])
              and np.array_equal(counts.cpu().numpy(), ref["counts"])
              and int(nrecv.item()) == ref["num_recv"])
        if non_expand:
            ok = ok and validate_non_expand(oracle, case, ref, last["expand"], last["recv_i"],
                                            last["recv_w"], last["out"], sample)
        else:
            ok = ok and validate_expand(oracle, case, ref, last["expand"], last["out"], sample, xb,
                                        dev)
        if not ok:
            print("bench: GPU results do not match the oracle; refusing to report", file=sys.stderr)
            sys.exit(1)
        cache = ("warm: one buffer set, steps back to back" if nsets == 1 else
                 f"cold: {nsets} buffer sets rotated, "
                 f"{(nsets - 1) * step_bytes / 1e6:.0f} MB of other traffic between uses of a set; "
                 f"{nx} copies of x rotated, {(nx - 1) * x_bytes / 1e6:.0f} MB of other x reads "
                 f"between uses of a copy")
        del sets, x_sets, last
        torch.cuda.empty_cache()
        return {"ms_per_step": ms_per_step, "us": us, "event_steps": n_ev,
                "launch": launch, "overlap": overlap, "cache": cache,
                "warmup_steps_run": n_load + n_warm}

    modes = ["cold"] if args.cold or args.cache == "cold" else \
        ["warm"] if args.cache == "warm" else ["warm", "cold"]
    runs = {}
    for m in modes:
        print(f"# {m} pass: {args.warmup} warm-up steps, {args.steps} timed steps, then "
              f"{max(20, args.event_steps)} instrumented steps", file=sys.stderr, flush=True)
        runs[m] = run_mode(m == "cold", m == modes[0])
    if args.workgroups > 0:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(stream, 0)
    plan_inside = (fused and not one_tile and not non_expand and not args.no_plan
                   and not args.workgroups)  # ep_layout_dispatch's own plan
    report(args, w, case, ref, runs, modes, copy_gbps, non_expand, use_plan or plan_inside, fused,
           one_tile)


class _CallRecorder:
    """Stands in for the loaded library: records each C call with its marshalled
    arguments instead of making it."""

    def __init__(self, L):
        self._L, self.calls = L, []

    def __getattr__(self, name):
        cfn = getattr(self._L, name)

        def record(*cargs):
            self.calls.append((cfn, cargs))
            return 0
        return record


def recorded_calls(B, issue):
    """The (C function, arguments) pairs the binding would call while `issue()`
    runs, so a timing loop can make the calls without the binding's per-call
    Python work (which exceeds a small kernel's own duration)."""
    L = B.lib()
    rec = _CallRecorder(L)
    B._LIB = rec
    try:
        issue()
    finally:
        B._LIB = L
    return rec.calls


GEMM_SHAPE = (8192, 7168, 2048)  # M, K, N: bf16 [M, K] x [K, N], about one step's duration


def overlap_gemm(torch, dev, step, step_ms: float, steps: int) -> dict:
    """A bf16 GEMM on its own stream: alone, then interleaved with the step.

    hidden_fraction = (step + gemm - both) / min(step, gemm): 1 when the
    shorter of the two runs entirely under the longer, 0 when they serialise.
    """
    M, K, N = GEMM_SHAPE
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn((M, K), device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn((K, N), device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty((M, N), device=dev, dtype=torch.bfloat16)
    gs = torch.cuda.Stream()  # default priority
    with torch.cuda.stream(gs):
        for _ in range(5):
            torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(gs):
        for _ in range(steps):
            torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    gemm_ms = (time.perf_counter() - t0) * 1e3 / steps
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
        with torch.cuda.stream(gs):
            torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    both_ms = (time.perf_counter() - t0) * 1e3 / steps
    hidden = (step_ms + gemm_ms - both_ms) / min(step_ms, gemm_ms)
    return {"gemm": f"bf16 [{M},{K}]x[{K},{N}] torch.matmul", "gemm_ms": round(gemm_ms, 4),
            "gemm_tflops": round(2 * M * K * N / (gemm_ms * 1e-3) / 1e12, 1),
            "step_ms": round(step_ms, 4), "both_ms": round(both_ms, 4),
            "hidden_fraction": round(hidden, 3)}


def copy_reference(torch, dev, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """GB/s (read + write) of torch's copy_ of nbytes of uint8 (16-byte vector accesses)."""
    a = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        b.copy_(a)
    ev[1].record()
    torch.cuda.synchronize()
    sec = ev[0].elapsed_time(ev[1]) * 1e-3 / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / sec / 1e9


def validate_non_expand(oracle, case, ref, recv_x, recv_i, recv_w, out, sample) -> bool:
    """Received rows, ids, weights in full; sampled output rows."""
    w = case.w
    n = ref["num_recv"]
    rx, _, ri, rw = oracle.dispatch_compact(case.x, case.topk_idx, ref["dst_slot"],
                                            ref["recv_src_metadata"], n, None, case.topk_weights)
    ok = np.array_equal(recv_x.cpu().numpy()[:n], rx)
    ok = ok and np.array_equal(recv_i.cpu().numpy()[:n], ri)
    ok = ok and np.array_equal(recv_w.cpu().numpy()[:n].view(np.uint32), rw.view(np.uint32))
    if w.out_dtype == 1:
        want = oracle.combine_compact_f32(case.y, ref["dst_slot"], ref["recv_src_metadata"], n)
        return ok and np.array_equal(out.cpu().numpy().view(np.uint32)[sample],
                                     want.view(np.uint32)[sample])
    want = oracle.combine_compact(case.y, ref["dst_slot"], ref["recv_src_metadata"], n)
    return ok and np.array_equal(out.cpu().numpy().view(np.uint16)[sample], want[sample])


def validate_expand(oracle, case, ref, expand, out, sample, xb, dev) -> bool:
    import torch

    w = case.w
    ok = True
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
    return bool(ok)


def mode_figures(w, nb, run, non_expand, workload) -> dict:
    """Throughput, per-kernel times and the dominant kernel's roofline of one cache mode."""
    total_bytes = sum(nb.values())
    ms = run["ms_per_step"]
    us = run["us"]
    value = total_bytes / (ms * 1e-3) / 1e9
    dc_us = us["dispatch"] + us["combine"]
    dc_gbps = (nb["dispatch"] + nb["combine"]) / (dc_us * 1e-6) / 1e9
    dom = max(("dispatch", "combine"), key=lambda k: us[k])
    achieved = nb[dom] / (us[dom] * 1e-6) / 1e9
    dom_name = dom + ("_compact" if non_expand else "")
    roofline = {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(workload, dom_name),
                "algorithmic_bytes_per_launch": nb[dom], "avg_launch_us": round(us[dom], 2),
                "samples": run["event_steps"]}
    return {"value": round(value, 1), "ms_per_step": round(ms, 4),
            "pct_of_peak": round(100 * value / HBM_PEAK_GBPS, 2),
            "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "dispatch_combine_GBps": round(dc_gbps, 1),
            "dispatch_combine_pct_of_peak": round(100 * dc_gbps / HBM_PEAK_GBPS, 2),
            "dispatch_combine_tokens_per_s": round(w.T / (dc_us * 1e-6), 1),
            "kernel_us": {k: round(v, 2) for k, v in us.items()},
            "roofline": roofline}


def report(args, w, case, ref, runs, modes, copy_gbps, non_expand, plan_used=False, fused=False,
           one_tile=True):
    n_valid = int((ref["dst_slot"] >= 0).sum())
    nb = algorithmic_bytes(w, n_valid, ref["num_recv"], args.path)
    main_run = runs[modes[0]]
    fig = mode_figures(w, nb, main_run, non_expand, w.name)
    result = {
        "metric": METRIC,
        "value": fig["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": fig["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAMES[w.dtype] if w.out_dtype == 0 else
                 f"{DTYPE_NAMES[w.dtype]}->{DTYPE_NAMES[w.out_dtype]}",
        "data": "synthetic",
        "config": {"workload": w.name, "tokens": w.T, "hidden": w.H, "experts": w.E, "topk": w.K,
                   "expert_alignment": w.A, "capacity_rows": w.cap, "routing": w.routing,
                   "dispatch_dtype": DTYPE_NAMES[w.dtype], "combine_dtype": DTYPE_NAMES[w.out_dtype],
                   "parallelism": "one GPU, all experts local", "path": args.path,
                   "dispatch_plan": plan_used,
                   "layout_read_ahead": bool(args.read_ahead and not fused),
                   "layout_dispatch": ((("one launch" if one_tile else "one call") +
                                        (" (ep_layout_dispatch_compact)" if non_expand
                                         else " (ep_layout_dispatch)"))
                                       if fused else "separate calls"),
                   "workgroup_cap": args.workgroups or None,
                   "cache": main_run["cache"], "launch": main_run["launch"]},
        **{k: fig[k] for k in ("pct_of_peak", "tokens_per_s", "dispatch_combine_GBps",
                               "dispatch_combine_pct_of_peak", "dispatch_combine_tokens_per_s")},
        "copy_reference_GBps": round(copy_gbps, 1),
        "dispatch_combine_pct_of_copy": round(100 * fig["dispatch_combine_GBps"] / copy_gbps, 2),
        "kernel_us": fig["kernel_us"],
        "warmup_steps_run": main_run["warmup_steps_run"],
        "warmup_detail": f"about {LOAD_MS:.0f} ms (at most {LOAD_MAX_STEPS} steps) of untimed "
                         f"steps queued back to back, then the {args.warmup} warm-up steps (more "
                         f"where cold mode rotates more buffer sets or x copies), then the timed "
                         f"steps, each after a synchronisation",
        "kernel_timing": f"HIP events around {main_run['event_steps']} back-to-back launches of "
                         f"each pass after {N_PRE_LAUNCHES} untimed ones, run right after the "
                         f"timed loop, each series queued after about {LOAD_MS:.0f} ms of untimed "
                         f"steps and a GPU spin of under 1 ms; mean per launch" +
                         ("; the fused call's time (layout included) is dispatch's" if fused
                          else ""),
        "algorithmic_bytes": nb,
        **({"overlap": main_run["overlap"]} if main_run["overlap"] else {}),
        "roofline": fig["roofline"],
    }
    for m in modes[1:]:
        sub = mode_figures(w, nb, runs[m], non_expand, w.name)
        sub["roofline"]["traffic"] = None  # counters are taken on the warm loop only
        result[m] = {**sub, "cache": runs[m]["cache"],
                     "warmup_steps_run": runs[m]["warmup_steps_run"]}
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(case, path=args.path)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
