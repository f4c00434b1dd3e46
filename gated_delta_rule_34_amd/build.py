"""Build the gfx950 HIP library ``libgdn.so`` in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled for gfx950 only and linked into one
shared library that exports the C ABI of ``include/gdn.h``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgdn.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# Per-file extras.  The fused kernels keep their MFMA accumulators in
# architectural VGPRs (they fit in 256 without spilling); the default
# accumulator-register form makes the compiler copy the state between the
# two register files around every VALU step.
FILE_FLAGS = {
    "gdn_fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "gdn2_fused.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, resource_usage: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if resource_usage and err:
        print(err, file=sys.stderr)
    return obj


def build(resource_usage: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, resource_usage), srcs))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="-v" in sys.argv))
