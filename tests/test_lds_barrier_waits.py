"""An s_barrier orders the waves of a workgroup, not their LDS traffic: a write
to LDS that another wave reads after the barrier must have completed before
the writer reaches it (s_waitcnt lgkmcnt(0)); on gfx950 the compiler places no
such wait in front of a barrier by itself.  This check compiles every kernel
source to gfx950 assembly and asserts, for each s_barrier, that every LDS
write between it and the previous barrier in the listing is followed by an
lgkmcnt(0) wait before the barrier."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_06_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _lgkm0(line):
    # s_waitcnt with lgkmcnt(0) named, or a bare immediate whose lgkmcnt field is 0
    if not line.startswith("s_waitcnt"):
        return False
    if "lgkmcnt(0)" in line:
        return True
    m = re.match(r"s_waitcnt\s+(0x[0-9a-fA-F]+|\d+)$", line)
    return bool(m) and ((int(m.group(1), 0) >> 8) & 0xF) == 0


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_lds_writes_complete_before_barriers(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    lines = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    pending = None  # last LDS write not yet waited for
    for l in lines:
        if not l or l.startswith("."):
            continue
        if l.endswith(":") and not l.startswith(".L"):  # a function starts
            pending = None
            continue
        if l.startswith("ds_write") or l.startswith("ds_store"):
            pending = l
        elif _lgkm0(l):
            pending = None
        elif l.startswith("s_barrier"):
            assert pending is None, f"{src}: LDS write not waited for before a barrier: {pending}"
