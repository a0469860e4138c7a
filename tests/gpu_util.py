"""Device-side helpers for the GPU tests: allocate, call the C ABI, read back.

Only marshalling lives here; every computation on the device runs in the
library's HIP kernels, reached through combine_ep_layout_amd.binding.
"""
import numpy as np
import torch

from combine_ep_layout_amd import binding as B
from combine_ep_layout_amd import inputs as I

DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def to_host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def dev_layout(idx_d: torch.Tensor, T: int, K: int, E: int, A: int, cap: int, stream=None,
               plan: bool = False, prefetch=None):
    """Run ep_layout; returns a dict of device tensors (with the dispatch plan if asked)."""
    counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    dst = torch.full((max(T, 1), K), -7, dtype=torch.int32, device=DEV)
    meta = torch.full((max(T, 1), K + 2), -7, dtype=torch.int32, device=DEV)
    nrecv = torch.full((1,), -7, dtype=torch.int32, device=DEV)
    wsb = B.ep_layout_workspace_bytes(T, K, E)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
    pl = torch.full((max(T * K, 1), 2), -9, dtype=torch.int32, device=DEV) if plan else None
    B.ep_layout(idx_d if T else None, T, K, E, A, cap, counts, offsets, dst if T else None,
                meta if T else None, nrecv, ws, wsb, stream, dispatch_plan=pl, prefetch=prefetch)
    out = {"counts": counts, "offsets": offsets, "dst_slot": dst[:T], "meta": meta[:T],
           "num_recv": nrecv}
    if plan:
        out["plan"] = pl[:T * K]
    return out


def layout_to_host(d):
    n = int(d["num_recv"].item())
    return {"counts": to_host(d["counts"]), "offsets": to_host(d["offsets"]),
            "dst_slot": to_host(d["dst_slot"]), "num_recv": n,
            "recv_src_metadata": to_host(d["meta"])[:n], "meta_full": to_host(d["meta"])}


class DeviceCase:
    """A Case uploaded to the GPU, with expand / output buffers allocated."""

    def __init__(self, case: I.Case, sentinel: int = 0x5A, with_y: bool = True):
        w = case.w
        self.w = w
        self.case = case
        self.idx = to_dev(case.topk_idx)
        self.wts = to_dev(case.topk_weights)
        self.x = to_dev(case.x)
        self.xs = to_dev(case.x_scales) if case.x_scales is not None else None
        self.y = to_dev(case.y) if (with_y and case.y is not None) else None
        elt = {I.BF16: 2, I.FP32: 4, I.FP8_E4M3: 1, I.FP4X2: 1}[w.dtype]
        self.row_bytes = w.H * elt
        self.expand_x = torch.full((w.cap, self.row_bytes), sentinel, dtype=torch.uint8, device=DEV)
        self.expand_s = (torch.full((w.cap, case.x_scales.shape[1]), -3.0, dtype=torch.float32,
                                    device=DEV) if self.xs is not None else None)
        self.expand_w = torch.full((w.cap,), -5.0, dtype=torch.float32, device=DEV)
        self.H_out = 2 * w.H if w.dtype == I.FP4X2 else w.H  # combine sees one value per element
        if w.out_dtype == I.FP32:
            self.out = torch.full((max(w.T, 1), self.H_out), float("nan"), dtype=torch.float32,
                                  device=DEV)
        else:
            self.out = torch.full((max(w.T, 1), self.H_out), 0x7FC1, dtype=torch.int16, device=DEV)
        self.sentinel = sentinel

    def layout(self, stream=None, plan=False, read_ahead=False):
        """ep_layout (with the dispatch plan if asked, and x as its read-ahead region if asked)."""
        w = self.w
        self.lay = dev_layout(self.idx, w.T, w.K, w.E, w.A, w.cap, stream, plan=plan,
                              prefetch=self.x if read_ahead else None)
        return self.lay

    def layout_dispatch(self, stream=None, weights=True, plan_workspace=False):
        """ep_layout_dispatch: the layout's outputs and the expand buffer in one call (with a
        workspace that holds a dispatch plan if asked)."""
        w = self.w
        T, K, E = w.T, w.K, w.E
        counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
        offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
        dst = torch.full((max(T, 1), K), -7, dtype=torch.int32, device=DEV)
        meta = torch.full((max(T, 1), K + 2), -7, dtype=torch.int32, device=DEV)
        nrecv = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        wsb = (B.ep_layout_dispatch_workspace_bytes(T, K, E) if plan_workspace
               else B.ep_layout_workspace_bytes(T, K, E))
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=DEV)
        B.ep_layout_dispatch(self.idx if T else None, T, K, E, w.A, w.cap, counts, offsets,
                             dst if T else None, meta if T else None, nrecv, ws, wsb,
                             self.x if T else None, self.xs, self.wts if weights else None, w.H,
                             w.dtype, self.expand_x, self.expand_s,
                             self.expand_w if weights else None, stream)
        self.lay = {"counts": counts, "offsets": offsets, "dst_slot": dst[:T], "meta": meta[:T],
                    "num_recv": nrecv}
        return self.lay

    def dispatch(self, stream=None, weights=True, plan=False):
        w = self.w
        B.ep_dispatch(self.x, self.xs, self.wts if weights else None, self.lay["dst_slot"], w.T,
                      w.H, w.K, w.dtype, w.cap, self.expand_x, self.expand_s,
                      self.expand_w if weights else None, stream,
                      dispatch_plan=self.lay["plan"] if plan else None)

    def combine(self, y=None, weights=True, bias=None, stream=None):
        w = self.w
        B.ep_combine(self.y if y is None else y, self.wts if weights else None, bias,
                     self.lay["dst_slot"], w.T, self.H_out, w.K, w.out_dtype, w.cap, self.out,
                     stream)
        return self.out[:w.T]
