"""The direct global->LDS loads are issued through inline assembly that sets
M0 (the LDS base) itself, so that the compiler neither tracks them as pending
LDS writes nor waits for them before unrelated LDS reads.  The compiler warns
that M0 is a reserved register: that is harmless only while the generated code
never keeps a value of its own in M0.  This check compiles every kernel source
to gfx950 assembly and asserts that each M0 reference is one of these
statement pairs: a write of M0 directly followed by the load that reads it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_06_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", sorted(f for f in os.listdir(CSRC) if f.endswith(".hip")))
def test_m0_only_feeds_direct_loads(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S",
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    lines = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    code = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    for i, l in enumerate(code):
        if not re.search(r"\bm0\b", l):
            continue
        assert l.startswith("s_mov_b32 m0,"), f"{src}: M0 used outside a direct load: {l}"
        nxt = code[i + 1] if i + 1 < len(code) else ""
        assert nxt.startswith("global_load_lds_dwordx4"), f"{src}: M0 write not followed by its load: {nxt}"
