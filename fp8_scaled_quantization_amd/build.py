"""Build the HIP library libfp8q.so for gfx950 with hipcc (cross-compiles without a GPU)."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8q.so")
SOURCES = ["capi.hip", "amax_history.hip", "quantize.hip", "gemm.hip", "next.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one object each) and link libfp8q.so (always recompiles)."""
    tag = "%d" % os.getpid()
    objs = [os.path.join(CSRC, s + ".%s.o" % tag) for s in SOURCES]
    cmds = [[HIPCC] + FLAGS + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    try:
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, out), s in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError("hipcc failed on %s:\n%s" % (s, out))
            if verbose and out.strip():
                print(out)
        tmp = LIB + ".tmp" + tag
        rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp])
        if rc != 0:
            raise RuntimeError("link failed:\n" + out)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
