"""Every fused-kernel instance compiles for gfx950 with no scratch memory (no
register spills): scratch reloads share the vector-memory counter with the
LDS-DMA, so a spill inside the step loop would serialise copy and math.  The
check compiles the fused kernel's device code with the library's flags and
reads the compiler's resource report (host only, no GPU)."""
import os
import re
import shutil
import subprocess

import pytest

from tile_sparse_mixed_amd import build as B

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_fused_kernel_instances_use_no_scratch(tmp_path):
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-c", "-x", "hip", os.path.join(B.CSRC, "k3_attn.hip"),
           "-o", str(tmp_path / "k3.o"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    text = r.stdout + r.stderr
    names = re.findall(r"Function Name: (\S+)", text)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
    k3 = [(n, s) for n, s in zip(names, scratch) if "k3_attn" in n]
    assert len(k3) >= 32, (len(names), len(scratch))   # D x NW x key block x SKIM x DUMP
    spills = [(n, s) for n, s in k3 if s != 0]
    assert not spills, spills
