"""Compile the HIP library ``libdsa.so`` in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("dsa_api.hip", "dsa_kernels.hip", "dsa_profile.hip", "dsa_probe.hip")]
HEADERS = [os.path.join(ROOT, "include", "dsa.h"), os.path.join(HERE, "csrc", "dsa_internal.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU forms stay off: all fp32 math goes through scalar forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: without it the characterization
    # kernels' accumulators are copied between AGPRs and VGPRs around every
    # MFMA step (the decode kernels use no MFMA; their code is unchanged)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Always recompiles; writes atomically so a loaded copy is never truncated."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include"), "-o", tmp] + SOURCES
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg:
        print(msg)
    os.replace(tmp, LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
