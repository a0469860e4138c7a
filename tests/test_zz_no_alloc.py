"""ep_layout_noalloc: the layout on the library's fixed scratch, against ep_layout.

For callers that cannot allocate device memory. Every output (counts,
offsets, slots, receive metadata, num_recv, dispatch plan) must equal what
ep_layout writes with a caller-owned workspace, bit for bit, on two calls in
a row, the second with a smaller batch: the scratch keeps the first call's
contents, which the second must not depend on. Sizes cover the two-launch
layout, the tile-scan layout (many tiles per expert), a workgroup cap whose
tiles loop, and a batch small enough to need no scratch; a batch whose
workspace exceeds the fixed scratch is rejected before any launch.
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
from tests.gpu_util import DEV, dev_layout, to_dev, to_host  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _noalloc_layout(idx_d, T, K, E, A, cap, stream):
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    dst = torch.full((max(T, 1), K), -7, dtype=torch.int32, device=DEV)
    meta = torch.full((max(T, 1), K + 2), -7, dtype=torch.int32, device=DEV)
    nrecv = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    plan = torch.full((max(T * K, 1), 2), -9, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()  # the fills ran on the default stream
    B.ep_layout_noalloc(idx_d, T, K, E, A, cap, counts, offsets, dst, meta, nrecv, stream,
                        dispatch_plan=plan)
    return {"counts": counts, "offsets": offsets, "dst_slot": dst[:T], "meta": meta[:T],
            "num_recv": nrecv, "plan": plan[:T * K]}


def _host(d):
    return {k: to_host(v) for k, v in d.items()}


# (first call, second smaller call, workgroup cap): (T, E, K, A, mask fraction)
PAIRS = [
    ("two-launch layout", (4096, 256, 8, 128, 0.0), (2500, 256, 8, 16, 0.05), 0),
    ("tile-scan layout", (20000, 1024, 8, 4, 0.02), (9000, 1024, 8, 1, 0.0), 0),
    ("capped, tiles loop", (6000, 256, 6, 8, 0.1), (3000, 64, 6, 2, 0.0), 7),
    ("scratch then none", (30000, 300, 4, 1, 0.0), (700, 300, 4, 32, 0.2), 0),
]


@pytest.mark.parametrize("name,first,second,wg_cap", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_layout_matches_ep_layout(name, first, second, wg_cap):
    s = torch.cuda.Stream()
    try:
        B.ep_set_workgroup_limit(s, wg_cap)
        for call, (T, E, K, A, mask) in enumerate((first, second)):
            need = B.ep_layout_workspace_bytes(T, K, E)
            _say(f"[noalloc] {name} call {call}: T={T} E={E} K={K} A={A} mask={mask} "
                 f"cap={wg_cap} scratch={need}")
            assert need <= B.EP_LAYOUT_SCRATCH_BYTES
            g = np.random.default_rng([T, E, K, 41])
            idx = I.routing_uniform(g, T, E, K)
            idx[g.random(idx.shape) < mask] = -1
            cap = T * K + E * (A - 1)
            idx_d = to_dev(idx)
            torch.cuda.synchronize()
            got = _noalloc_layout(idx_d, T, K, E, A, cap, s)
            want = dev_layout(idx_d, T, K, E, A, cap, stream=s, plan=True)
            s.synchronize()
            got, want = _host(got), _host(want)
            for k in ("counts", "offsets", "dst_slot", "num_recv", "plan"):
                assert np.array_equal(got[k], want[k]), f"{name} call {call}: {k}"
            n = int(want["num_recv"][0])
            assert np.array_equal(got["meta"][:n], want["meta"][:n]), f"{name} call {call}: meta"
            assert np.all(got["meta"][n:] == -7), "rows past num_recv stay untouched"
            ref = oracle.layout(idx, E, A)
            assert np.array_equal(got["dst_slot"], ref["dst_slot"])
            assert np.array_equal(got["offsets"], ref["offsets"])
    finally:
        torch.cuda.synchronize()
        B.ep_set_workgroup_limit(s, 0)


def test_noalloc_rejects_batches_beyond_the_scratch():
    T, K, E = 40000, 8, 1024
    need = B.ep_layout_workspace_bytes(T, K, E)
    assert need > B.EP_LAYOUT_SCRATCH_BYTES
    idx = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    outs = [torch.full(n, -7, dtype=torch.int32, device=DEV)
            for n in ((E,), (E + 1,), (T, K), (T, K + 2), (1,))]
    torch.cuda.synchronize()
    with pytest.raises(B.EpError) as ei:
        B.ep_layout_noalloc(idx, T, K, E, 1, T * K, *outs)
    assert ei.value.code == B.EP_EINVAL and "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert all(bool((o == -7).all()) for o in outs), "nothing was launched"
