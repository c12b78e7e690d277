"""Build libdsfp8.so for gfx950 with hipcc (in-tree, no JIT cache).

``python -m block_scaled_fp8_act_amd.build`` compiles every source under
``csrc/`` into ``block_scaled_fp8_act_amd/libdsfp8.so``.  hipcc cross-compiles
the device code, so this runs on a machine without a GPU.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsfp8.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "quant.hip", "gemm.hip", "moe.hip"]

COMMON = [
    "-O3", "-fPIC", "-std=c++17", "-Wall",
    f"-I{os.path.join(ROOT, 'include')}",
]
# Device code: gfx950 only, correctly rounded fp32 division (hipcc's default,
# stated explicitly), no packed-fp32 instruction selection.
DEVICE = [
    f"--offload-arch={ARCH}",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: the GEMMs rescale every MFMA result on the VALU,
    # which cannot read AGPRs directly.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return exe


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c"] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + ["-x", "hip"]
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    cmd += [os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r


def build(verbose=False):
    """Compile all sources and link the shared library; raise on any error."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = []
    for src, obj, r in results:
        if verbose and (r.stdout or r.stderr):
            print(r.stdout + r.stderr, file=sys.stderr)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
