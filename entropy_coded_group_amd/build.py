"""Build libecco.so in-tree with hipcc for gfx950.

    python -m entropy_coded_group_amd.build

Every call recompiles.  Objects go to entropy_coded_group_amd/_build/, the
shared library to entropy_coded_group_amd/libecco.so.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libecco.so")
ARCH = "gfx950"

SOURCES = ["ecco_tables.cpp", "ecco_train.cpp", "ecco_kernels.hip", "ecco_gemv.hip", "ecco_attn.hip",
           "ecco_spec.hip"]

# -ffp-contract=off: every float step that decides an output bit is a single
# IEEE operation (no fused multiply-add).  Packed FP32 instructions are
# disabled for device code.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(os.path.dirname(PKG), "include")]
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + COMMON + ["-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE
    else:
        cmd += ["-pthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the device target feature: harmless notice
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and "is not a recognized feature" not in l]
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (" ".join(cmd), "\n".join(lines)))
    if verbose and lines:
        print("\n".join(lines))
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-pthread", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
