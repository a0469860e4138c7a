"""The oracle is plain host C: no HIP header, no code shared with the GPU library."""
import os
import re
import subprocess

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_builds_with_plain_gcc(tmp_path):
    out = str(tmp_path / "liboracle_check.so")
    obuild.build(cc="gcc", out=out)
    assert os.path.getsize(out) > 0


def test_oracle_includes_only_libc_headers():
    src = open(obuild.SRC).read()
    incs = re.findall(r'#\s*include\s*[<"]([^>"]+)[>"]', src)
    assert set(incs) <= {"stdint.h", "stdlib.h", "string.h"}, incs


def test_oracle_and_gpu_library_share_no_code():
    pkg = os.path.join(ROOT, "combine_ep_layout_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp", ".c")):
                text = open(os.path.join(dirpath, f), errors="ignore").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "ep_oracle" not in text, f
    ora = os.path.join(ROOT, "oracle")
    for f in os.listdir(ora):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ora, f)).read()
            assert "combine_ep_layout_amd" not in text, f
            assert "csrc" not in text, f
