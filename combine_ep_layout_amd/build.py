"""Build libep_mi355x.so (the C-ABI library) for gfx950 with hipcc.

Every translation unit is compiled for gfx950 only, with binary32 packed
math disabled (-packed-fp32-ops), then linked into one shared library next
to this file. Objects go to <repo>/_build/.

`python build.py --asan-host` instead builds libep_mi355x_asan.so with
AddressSanitizer on the host code only (device code is unchanged); load it
with the clang ASan runtime preloaded to check the C ABI's host paths.

build_small_launch() builds libep_mi355x_small_launch.so, a test build in
which one launch of the one-unit-per-wave kernels covers at most
SMALL_LAUNCH_UNITS units, so that small GPU tests run the paths that split
large inputs over several launches (or fall back to looping kernels).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libep_mi355x.so")

SOURCES = ["ep_capi.cpp", "ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip", "ep_padding.hip",
           "ep_compact.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics"]


ASAN_HOST = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LIB = os.path.join(PKG, "libep_mi355x_asan.so")

SMALL_LAUNCH_UNITS = 4160
SMALL_LAUNCH_LIB = os.path.join(PKG, "libep_mi355x_small_launch.so")
SMALL_LAUNCH_SOURCES = ("ep_dispatch.hip", "ep_compact.hip", "ep_combine.hip")  # its users


def _compile(src: str, extra=(), tag: str = "") -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + tag + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip", *DEVICE, *COMMON, *extra, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *COMMON, *extra, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(out: str = LIB, extra=(), jobs: int = 4, verbose: bool = False,
          asan_host: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    if asan_host:
        extra = (*extra, *ASAN_HOST)
        out = ASAN_LIB if out == LIB else out
    tag = ".asan" if asan_host else ""
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, tag), SOURCES))
    tmp = out + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address"] if asan_host else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(out)
    return out


def build_small_launch(jobs: int = 4, verbose: bool = False) -> str:
    """The test build: the library with EP_MAX_LAUNCH_UNITS = SMALL_LAUNCH_UNITS. Reuses the
    objects of build() for the sources that do not read the limit (call build() first)."""
    os.makedirs(BUILD, exist_ok=True)
    extra = (f"-DEP_MAX_LAUNCH_UNITS={SMALL_LAUNCH_UNITS}",)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        small = dict(zip(SMALL_LAUNCH_SOURCES,
                         ex.map(lambda s: _compile(s, extra, ".small"), SMALL_LAUNCH_SOURCES)))
    objs = [small.get(s) or os.path.join(BUILD, s + ".o") for s in SOURCES]
    tmp = SMALL_LAUNCH_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SMALL_LAUNCH_LIB)
    if verbose:
        print(SMALL_LAUNCH_LIB)
    return SMALL_LAUNCH_LIB


if __name__ == "__main__":
    args = sys.argv[1:]
    asan = "--asan-host" in args
    build(verbose=True, extra=[a for a in args if a != "--asan-host"], asan_host=asan)
