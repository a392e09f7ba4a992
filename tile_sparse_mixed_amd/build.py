"""Build the tattn shared library (libtattn.so) in-tree for gfx950 with hipcc.

    python -m tile_sparse_mixed_amd.build
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libtattn.so")
# the fused pass is split into one translation unit per key-block size
# (k3_bk*.hip), compiled in parallel
K3_UNITS = ["k3_bk64.hip", "k3_bk16.hip", "k3_bk8.hip", "k3_bk4.hip", "k3_bk2.hip", "k3_bk1.hip"]
SOURCES = ["k1_pool.hip", "k2_router.hip", "k3_attn.hip", *K3_UNITS, "tattn_host.cpp"]
# Packed fp32 instructions are kept out of every kernel: the compiler would
# otherwise form v_pk_* fp32 ops from float and float2 code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object (in parallel, `jobs` at a time; 0:
    up to the CPU count, at most 8) and link libtattn.so."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = tempfile.mkdtemp(prefix="tattn_build_")
    try:
        cflags = [f for f in FLAGS if f != "-shared"]
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(objdir, src + ".o")
            objs.append(obj)
            cmds.append([hipcc, *cflags, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj])
        n = jobs or min(8, os.cpu_count() or 1)
        with ThreadPoolExecutor(max_workers=n) as ex:
            for f in [ex.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = OUT + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, OUT)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
