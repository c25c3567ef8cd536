"""Build libgdn.so (gfx950) in-tree with hipcc.

    python -m gated_delta_rule_29_amd.build

Every .hip file under csrc/ is compiled for gfx950 only (one hipcc process per file, run in
parallel) and linked into gated_delta_rule_29_amd/libgdn.so.  Packed-fp32 instruction selection is disabled for all
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


# Extra code-generation flags per source.  The state scan keeps its matrix-core accumulators in
# ordinary VGPRs: its products feed vector arithmetic directly, and accumulator registers
# would cost a copy per element.
FILE_FLAGS = {
    "gdn_scan16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}

COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-result"]

# The host pass does not know the packed-fp32 target feature and says so; drop that noise.
_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (res.stderr + res.stdout).splitlines() if _NOISE not in l)
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip (in parallel) and link them into libgdn.so; returns its path."""
    from concurrent.futures import ThreadPoolExecutor

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tag = "%d" % os.getpid()
    objs = [os.path.join(CSRC, "_obj_%s_%s.o" % (tag, os.path.basename(s)[:-4])) for s in srcs]
    inc = ["-I", os.path.join(HERE, "..", "include")]
    cmds = [[hipcc(), *COMMON, *FILE_FLAGS.get(os.path.basename(s), []), *inc, "-c", s, "-o", o]
            for s, o in zip(srcs, objs)]
    tmp = LIB + ".tmp" + tag
    try:
        with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, msgs) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd))
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + msgs)
            if verbose and msgs.strip():
                print(msgs)
        rc, msgs = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + msgs)
        os.replace(tmp, LIB)
    finally:
        for o in objs + [tmp]:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
