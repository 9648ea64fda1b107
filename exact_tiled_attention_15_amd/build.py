"""Build libattn.so from the HIP sources in csrc/ for gfx950 (in-tree).

Every source is compiled by hipcc for --offload-arch=gfx950 with packed fp32
VALU instructions disabled, and the objects are linked into one shared
library next to this file.  Object files go to <repo>/_build/.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
BUILD_DIR = os.path.join(REPO_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
SOURCES = ["fwd_bf16.hip", "fwd_fp8.hip", "fwd_f32.hip", "merge.hip", "bwd_bf16.hip", "w4a16.hip", "mfma_probe.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
# Kernels whose matrix accumulators do not all fit in the architectural VGPRs:
# without this option the compiler keeps MFMA results in AGPRs and copies the
# live accumulators out and back around every other product (about 190
# v_accvgpr moves per key tile in the dK/dV kernel); with it the products
# accumulate in VGPRs directly and the long-lived sums alone sit in AGPRs.
EXTRA_FLAGS = {
    "bwd_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "fwd_f32.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    """Compile every source and link libattn.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".", "_") + ".o")
        objs.append(obj)
        cmds.append([HIPCC, *COMMON_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for msg in ex.map(_run, cmds):
            if verbose and msg.strip():
                print(msg, file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
