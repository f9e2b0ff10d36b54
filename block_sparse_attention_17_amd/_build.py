"""Compile the HIP sources into the in-tree shared library ``libsvsa.so`` (gfx950).

Run as ``python block_sparse_attention_17_amd/_build.py`` (as a script: the
package itself refuses to import until the library exists).  Objects go to
``_build/`` next to the sources; the library lands inside the package.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
OUT = os.path.join(PKG, "libsvsa.so")
BUILD = os.path.join(PKG, "_build")
ARCH = os.environ.get("SVSA_OFFLOAD_ARCH", "gfx950")

SOURCES = ["api.cpp", "permute.hip", "pool.hip", "mask.hip", "stripe.hip", "attn.hip",
           "cluster.hip"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsvsa.so)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", f"-I{INCLUDE}",
            # keep the compiler from forming packed fp32 instructions from float code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-result", "-Wno-unused-variable"]


# Per-file flags.  The attention kernel never produces NaN (padded keys are
# -inf, every row has a finite maximum), so IEEE NaN quieting before each
# v_max_f32 is dropped there.
EXTRA = {"attn.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + EXTRA.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]  # host-only file; compiled by hipcc to share the runtime headers
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
