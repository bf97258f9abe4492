"""Build libmla.so (all HIP sources under csrc/) for gfx950 with hipcc.

Usage: python -m compressed_kv_cache_mla_amd.build  (or build() from Python).
The library is written next to this file so that it travels with the tree.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
ARCH = os.environ.get("MLA_OFFLOAD_ARCH", "gfx950")

# -packed-fp32-ops: keep hipcc from forming packed fp32 VALU ops.
# -fno-honor-nans: no NaN inputs are expected (infinities still are: masked
# scores are -inf), so fmaxf needs no quieting of its operands.
# -amdgpu-mfma-vgpr-form: MFMA builtins accumulate in VGPRs; the decode
# kernel's long-lived accumulators are kept in AGPRs by inline asm, so the
# short-lived score accumulators no longer displace them.
HIPCC_FLAGS = ["-O3", "-std=c++17", "-fno-honor-nans", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form",
               "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmla.so)")


def build(verbose: bool = False, extra_flags=None, out: str = LIB) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
    print("built", LIB)
