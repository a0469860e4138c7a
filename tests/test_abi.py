"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host with the documented codes (no GPU needed: every check
runs before anything is enqueued, and no test here makes a compute call)."""
import ctypes
import os
import re

import pytest

from combine_ep_layout_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep_mi355x.h")
FAKE = 1 << 20  # a 16-byte aligned, never dereferenced address
ODD = FAKE + 4  # misaligned for rows


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B.LIB_PATH):
        from combine_ep_layout_amd import build
        build.build()
    return B.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbols():
    assert declared_functions() == sorted(B.SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (EP_[A-Z0-9_]+) \(?(-?\d+)\)?", text))
    for k, v in consts.items():
        assert getattr(B, k) == int(v), k


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        B.lib(str(tmp_path / "nope.so"))


def test_supported_set(L):
    assert B.ep_supported(0, 0, 8, 0)
    assert B.ep_supported(1, 7168, 8, B.EP_BF16)
    assert B.ep_supported(1, 7168, 8, B.EP_FP8_E4M3)
    assert B.ep_supported(2, 7168, 8, B.EP_BF16)
    assert B.ep_supported(2, 7168, 8, B.EP_FP32)
    assert B.ep_supported(1, 7168, 8, B.EP_FP32)
    assert B.ep_supported(1, 3584, 8, B.EP_FP4X2)      # hidden counts bytes for fp4x2
    assert not B.ep_supported(1, 7168, 8, B.EP_FP4X2)
    assert not B.ep_supported(2, 7168, 8, B.EP_FP8_E4M3)
    assert not B.ep_supported(1, 7168, 3, B.EP_BF16)
    assert not B.ep_supported(1, 1000, 8, B.EP_BF16)
    assert not B.ep_supported(7, 7168, 8, B.EP_BF16)


def test_workspace_bytes(L):
    assert B.ep_layout_workspace_bytes(64, 2, 16) == 0          # one tile: no workspace
    assert B.ep_layout_workspace_bytes(1024, 8, 256) == 0       # single-launch multi-tile path
    assert B.ep_layout_workspace_bytes(4096, 8, 256) >= 32 * 257 * 4  # two-launch path
    assert B.ep_layout_workspace_bytes(-1, 8, 256) == 0
    assert B.ep_layout_workspace_bytes(10, 8, 5000) == 0


def _code(fn, *a):
    with pytest.raises(B.EpError) as ei:
        fn(*a)
    assert B.ep_last_error() and str(ei.value)
    return ei.value.code


def lay(T=4096, K=8, E=256, A=128, cap=65280, ws=FAKE, wsb=1 << 20, idx=FAKE, counts=FAKE):
    return (idx, T, K, E, A, cap, counts, FAKE, FAKE, FAKE, FAKE, ws, wsb)


def test_layout_dispatch_workspace_bytes(L):
    """The fused call's plan-sized workspace: the layout's, rounded up to 256 bytes, plus
    8 bytes per entry; 0 for out-of-range arguments."""
    for T, K, E in [(64, 2, 16), (4096, 8, 256), (20000, 8, 1024), (1, 1, 1), (0, 8, 256)]:
        base = B.ep_layout_workspace_bytes(T, K, E)
        assert B.ep_layout_dispatch_workspace_bytes(T, K, E) == -(-base // 256) * 256 + T * K * 8
    assert B.ep_layout_dispatch_workspace_bytes(-1, 8, 256) == 0
    assert B.ep_layout_dispatch_workspace_bytes(16, 65, 256) == 0
    assert B.ep_layout_dispatch_workspace_bytes(16, 8, 1025) == 0


def test_layout_rejections(L):
    assert _code(B.ep_layout, *lay(T=-1)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(K=0)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(K=65)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(E=0)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(E=1025)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(A=0)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(cap=65279)) == B.EP_ECAPACITY
    assert _code(B.ep_layout, *lay(K=3, cap=1 << 20)) == B.EP_EUNSUPPORTED
    big = dict(T=32768, cap=32768 * 8 + 256 * 127)                   # needs a workspace
    assert _code(B.ep_layout, *lay(ws=None, **big)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(wsb=16, **big)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(ws=ODD, **big)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(idx=None)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(counts=None)) == B.EP_EINVAL
    assert _code(B.ep_layout, *lay(T=1 << 28, cap=1 << 40)) == B.EP_EINVAL  # T*K overflows int32
    with pytest.raises(B.EpError) as ei:  # a read-ahead region needs a pointer
        B.ep_layout(*lay(), prefetch=0, prefetch_bytes=1 << 20)
    assert ei.value.code == B.EP_EINVAL and "prefetch" in str(ei.value)
    with pytest.raises(B.EpError) as ei:  # read as 4-byte words
        B.ep_layout(*lay(ws=None, wsb=0, T=64, K=2, E=16, A=1, cap=128), prefetch=FAKE + 2,
                    prefetch_bytes=4096)
    assert ei.value.code == B.EP_EINVAL and "prefetch" in str(ei.value)
    plan_4 = FAKE + 4  # (entry, slot) pairs need 8-byte alignment
    with pytest.raises(B.EpError) as ei:
        B.ep_layout(*lay(), dispatch_plan=plan_4)
    assert ei.value.code == B.EP_EINVAL and "dispatch_plan" in str(ei.value)


def disp(x=FAKE, xs=None, dst=FAKE, T=4096, H=7168, K=8, dt=B.EP_BF16, cap=65280, X=FAKE, Xs=None):
    return (x, xs, None, dst, T, H, K, dt, cap, X, Xs, None)


def test_fp8_without_scales_passes_the_checks(L):
    """fp8 rows may travel without scale rows (the header's reading: the payload is
    bytes either way): a NULL x_scales passes every argument check, and so does a
    hidden size that is not a multiple of 128 then. An uncompiled topk (3) stops
    each call at the capability gate, after those checks and before any launch."""
    for H in (7168, 7184):
        assert _code(B.ep_dispatch, *disp(dt=B.EP_FP8_E4M3, H=H, K=3)) == B.EP_EUNSUPPORTED
    # with scale rows, hidden must be a multiple of 128 values
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP8_E4M3, H=7184, K=3, xs=FAKE, Xs=FAKE)) == \
        B.EP_EINVAL


def test_dispatch_rejections(L):
    assert _code(B.ep_dispatch, *disp(H=7169)) == B.EP_EINVAL           # 16-byte rows
    assert _code(B.ep_dispatch, *disp(H=7000)) == B.EP_EUNSUPPORTED     # aligned but not compiled
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP8_E4M3, xs=FAKE)) == B.EP_EINVAL  # one scale pointer
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP8_E4M3, Xs=FAKE)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP8_E4M3, H=7184, xs=FAKE, Xs=FAKE)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP4X2, H=3616, xs=FAKE, Xs=FAKE)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(xs=FAKE, Xs=FAKE)) == B.EP_EINVAL  # scales for bf16
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP32, xs=FAKE, Xs=FAKE)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP4X2)) == B.EP_EUNSUPPORTED   # 7168 bytes not compiled
    assert _code(B.ep_dispatch, *disp(dt=B.EP_FP32, H=7172)) == B.EP_EUNSUPPORTED
    assert _code(B.ep_dispatch, *disp(dt=9)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(x=ODD)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(X=None)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(cap=-1)) == B.EP_EINVAL
    assert _code(B.ep_dispatch, *disp(K=5)) == B.EP_EUNSUPPORTED
    with pytest.raises(B.EpError) as ei:
        B.ep_dispatch(*disp(), dispatch_plan=FAKE + 4)
    assert ei.value.code == B.EP_EINVAL and "plan" in str(ei.value)


def lay_disp(T=128, K=8, E=256, A=1, cap=1024, x=FAKE, xs=None, H=7168, dt=B.EP_BF16, X=FAKE,
             Xs=None):
    return (FAKE, T, K, E, A, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, x, xs, None, H, dt,
            X, Xs, None)


def test_layout_dispatch_rejections(L):
    """The fused call applies ep_layout's and ep_dispatch's checks (nothing is launched)."""
    assert _code(B.ep_layout_dispatch, *lay_disp(K=0)) == B.EP_EINVAL
    assert _code(B.ep_layout_dispatch, *lay_disp(E=1025)) == B.EP_EINVAL
    assert _code(B.ep_layout_dispatch, *lay_disp(cap=1023)) == B.EP_ECAPACITY
    assert _code(B.ep_layout_dispatch, *lay_disp(K=3, cap=1 << 20)) == B.EP_EUNSUPPORTED
    assert _code(B.ep_layout_dispatch, *lay_disp(H=7169)) == B.EP_EINVAL
    assert _code(B.ep_layout_dispatch, *lay_disp(H=7000)) == B.EP_EUNSUPPORTED
    assert _code(B.ep_layout_dispatch, *lay_disp(dt=9)) == B.EP_EINVAL
    assert _code(B.ep_layout_dispatch, *lay_disp(xs=FAKE, Xs=FAKE)) == B.EP_EINVAL  # bf16 scales
    assert _code(B.ep_layout_dispatch, *lay_disp(x=ODD)) == B.EP_EINVAL
    assert _code(B.ep_layout_dispatch, *lay_disp(X=None)) == B.EP_EINVAL
    assert "ep_layout_dispatch" in B.ep_last_error()


def lay_disp_c(T=128, K=8, E=256, A=1, cap=1024, x=FAKE, xs=None, w=None, H=7168, dt=B.EP_BF16,
               rx=FAKE, rs=None, ri=FAKE, rw=None):
    return (FAKE, T, K, E, A, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, x, xs, w, H, dt,
            rx, rs, ri, rw)


def test_layout_dispatch_compact_rejections(L):
    """The fused non-expand call applies ep_layout's and ep_dispatch_compact's checks
    (nothing is launched)."""
    f = B.ep_layout_dispatch_compact
    assert _code(f, *lay_disp_c(K=0)) == B.EP_EINVAL
    assert _code(f, *lay_disp_c(E=1025)) == B.EP_EINVAL
    assert _code(f, *lay_disp_c(cap=1023)) == B.EP_ECAPACITY
    assert _code(f, *lay_disp_c(K=3, cap=1 << 20)) == B.EP_EUNSUPPORTED
    assert _code(f, *lay_disp_c(H=7169)) == B.EP_EINVAL  # 14,338 bytes per row
    assert _code(f, *lay_disp_c(dt=9)) == B.EP_EINVAL
    assert _code(f, *lay_disp_c(xs=FAKE, rs=FAKE)) == B.EP_EINVAL  # scales with bf16 rows
    assert _code(f, *lay_disp_c(dt=B.EP_FP8_E4M3, xs=FAKE)) == B.EP_EINVAL  # scales go together
    assert _code(f, *lay_disp_c(x=ODD)) == B.EP_EINVAL
    assert _code(f, *lay_disp_c(rx=None)) == B.EP_EINVAL
    assert _code(f, *lay_disp_c(ri=None)) == B.EP_EINVAL
    assert _code(f, *lay_disp_c(w=FAKE)) == B.EP_EINVAL  # weights without recv_topk_weights
    assert "ep_layout_dispatch_compact" in B.ep_last_error()


def comb(y=FAKE, dst=FAKE, T=4096, H=7168, K=8, dt=B.EP_BF16, cap=65280, out=FAKE, bias=None):
    return (y, None, bias, dst, T, H, K, dt, cap, out)


def test_combine_rejections(L):
    assert _code(B.ep_combine, *comb(dt=B.EP_FP8_E4M3)) == B.EP_EINVAL  # byte dtypes cannot be summed
    assert _code(B.ep_combine, *comb(dt=B.EP_FP4X2)) == B.EP_EINVAL
    assert _code(B.ep_combine, *comb(dt=B.EP_FP32, H=7172)) == B.EP_EUNSUPPORTED
    assert _code(B.ep_combine, *comb(dt=5)) == B.EP_EINVAL
    assert _code(B.ep_combine, *comb(H=7172)) == B.EP_EINVAL
    assert _code(B.ep_combine, *comb(H=7176)) == B.EP_EUNSUPPORTED
    assert _code(B.ep_combine, *comb(out=ODD)) == B.EP_EINVAL
    assert _code(B.ep_combine, *comb(bias=ODD)) == B.EP_EINVAL
    assert _code(B.ep_combine, *comb(y=None)) == B.EP_EINVAL
    assert _code(B.ep_combine, *comb(K=0)) == B.EP_EINVAL


def test_zero_padding_rejections(L):
    ok = dict(x=FAKE, rb=14336, s=None, sc=0, w=None, c=FAKE, o=FAKE, E=256, A=128, cap=65280)

    def zp(**kw):
        a = {**ok, **kw}
        return (a["x"], a["rb"], a["s"], a["sc"], a["w"], a["c"], a["o"], a["E"], a["A"], a["cap"])
    assert _code(B.ep_zero_padding, *zp(rb=14330)) == B.EP_EINVAL
    assert _code(B.ep_zero_padding, *zp(rb=0)) == B.EP_EINVAL
    assert _code(B.ep_zero_padding, *zp(E=0)) == B.EP_EINVAL
    assert _code(B.ep_zero_padding, *zp(A=0)) == B.EP_EINVAL
    assert _code(B.ep_zero_padding, *zp(x=None)) == B.EP_EINVAL
    assert _code(B.ep_zero_padding, *zp(x=ODD)) == B.EP_EINVAL
    assert _code(B.ep_zero_padding, *zp(sc=56)) == B.EP_EINVAL          # scale columns without a pointer
    assert _code(B.ep_zero_padding, *zp(c=None)) == B.EP_EINVAL


def test_compact_rejections(L):
    def dc(**kw):
        a = dict(x=FAKE, xs=None, idx=FAKE, w=None, dst=FAKE, meta=FAKE, n=FAKE, T=4096, H=7168, K=8,
                 dt=B.EP_BF16, rx=FAKE, rs=None, ri=FAKE, rw=None)
        a.update(kw)
        return tuple(a.values())
    assert _code(B.ep_dispatch_compact, *dc(H=7169)) == B.EP_EINVAL
    assert _code(B.ep_dispatch_compact, *dc(xs=FAKE)) == B.EP_EINVAL       # scales without recv_scales
    assert _code(B.ep_dispatch_compact, *dc(xs=FAKE, rs=FAKE)) == B.EP_EINVAL  # scales with bf16
    assert _code(B.ep_dispatch_compact, *dc(meta=None)) == B.EP_EINVAL
    assert _code(B.ep_dispatch_compact, *dc(w=FAKE)) == B.EP_EINVAL        # weights without a destination
    assert _code(B.ep_dispatch_compact, *dc(rx=ODD)) == B.EP_EINVAL
    assert _code(B.ep_dispatch_compact, *dc(dt=7)) == B.EP_EINVAL

    def cc(**kw):
        a = dict(y=FAKE, b=None, dst=FAKE, meta=FAKE, n=FAKE, T=4096, H=7168, K=8, dt=B.EP_BF16, out=FAKE)
        a.update(kw)
        return tuple(a.values())
    assert _code(B.ep_combine_compact, *cc(dt=B.EP_FP8_E4M3)) == B.EP_EINVAL
    assert _code(B.ep_combine_compact, *cc(dt=7)) == B.EP_EINVAL
    assert _code(B.ep_combine_compact, *cc(H=7172)) == B.EP_EINVAL
    assert _code(B.ep_combine_compact, *cc(H=7170, dt=B.EP_FP32)) == B.EP_EINVAL  # 28,680 bytes
    assert _code(B.ep_combine_compact, *cc(n=None)) == B.EP_EINVAL
    assert _code(B.ep_combine_compact, *cc(b=ODD)) == B.EP_EINVAL


def test_workgroup_limit_host_side(L):
    assert _code(B.ep_set_workgroup_limit, FAKE, -1) == B.EP_EINVAL
    B.ep_set_workgroup_limit(FAKE, 0)  # clearing a cap that was never set is fine
    assert B.ep_get_workgroup_limit(FAKE) == 0
    assert B.ep_get_workgroup_limit(None) == 0


def test_layout_noalloc_host_rejections(L):
    """Checks that ep_layout_noalloc makes before touching any device."""
    def na(T=64, K=2, E=16, A=1, cap=128, idx=FAKE, counts=FAKE):
        return (idx, T, K, E, A, cap, counts, FAKE, FAKE, FAKE, FAKE)
    assert _code(B.ep_layout_noalloc, *na(T=-1)) == B.EP_EINVAL
    assert _code(B.ep_layout_noalloc, *na(K=65)) == B.EP_EINVAL
    assert _code(B.ep_layout_noalloc, *na(E=1025)) == B.EP_EINVAL
    assert _code(B.ep_layout_noalloc, *na(cap=127)) == B.EP_ECAPACITY  # one tile: no scratch
    assert _code(B.ep_layout_noalloc, *na(counts=None)) == B.EP_EINVAL
    T, K, E = 40000, 8, 1024  # 10 MB of workspace, above the fixed 8 MiB
    assert B.ep_layout_workspace_bytes(T, K, E) > B.EP_LAYOUT_SCRATCH_BYTES
    with pytest.raises(B.EpError) as ei:
        B.ep_layout_noalloc(*na(T=T, K=K, E=E, cap=T * K))
    assert ei.value.code == B.EP_EINVAL and "scratch" in str(ei.value)
