"""Build libgdn.so (gfx950) in-tree with hipcc.

    python -m gated_delta_rule_29_amd.build

Every .hip file under csrc/ is compiled for gfx950 only and linked into
gated_delta_rule_29_amd/libgdn.so.  Packed-fp32 instruction selection is disabled for all
device code (-packed-fp32-ops): the compiler then emits scalar fp32 arithmetic only.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile and link every csrc/*.hip into libgdn.so; returns the library path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-result", "-I", os.path.join(HERE, "..", "include"),
           *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 target feature and says so; drop that noise.
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stderr + res.stdout).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msgs)
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
