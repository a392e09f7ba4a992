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


def _report(unit, tmp_path):
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-c", "-x", "hip", os.path.join(B.CSRC, unit),
           "-o", str(tmp_path / (unit + ".o")), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout + r.stderr


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_fused_kernel_instances_use_no_scratch(tmp_path):
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        texts = list(ex.map(lambda u: _report(u, tmp_path), B.K3_UNITS))
    k3 = []
    for text in texts:
        names = re.findall(r"Function Name: (\S+)", text)
        scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", text)]
        assert len(names) == len(scratch), (len(names), len(scratch))
        k3 += [(n, s) for n, s in zip(names, scratch) if "k3_attn" in n]
    # D x NW x DUMP x six key-block sizes x (three tiers, with SKIM, refined low tier)
    assert len(k3) == 2 * 2 * 2 * 6 * 3, len(k3)
    spills = [(n, s) for n, s in k3 if s != 0]
    assert not spills, spills
