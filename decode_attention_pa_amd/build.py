"""Builds libpa_decode.so (gfx950) in-tree with hipcc.

The sources are compiled as separate translation units in parallel (the
matrix-core kernels of each head dim in their own unit) and linked into one
shared library.

Usage: python -m decode_attention_pa_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpa_decode.so")
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in
           ("pa_decode.hip", "pa_mfma_d64.hip", "pa_mfma_d128.hip", "pa_mfma_d256.hip",
            "pa_wave_kernels.hip")]
HEADERS = [os.path.join(ROOT, "include", "pa_decode.h")] + [
    os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in VGPRs: the online-softmax rescale and the
    # final normalisation then run on them in place, without AGPR copies
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def command(out: str = LIB, extra=()) -> list[str]:
    """One-step build command of the whole library (all sources, one hipcc)."""
    return [hipcc(), *FLAGS, "-shared", *extra, *SOURCES, "-o", out]


def _run(cmds, verbose):
    noise = "is not a recognized feature for this target"
    procs = []
    for cmd in cmds:
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    errs = []
    for cmd, p in procs:
        _, err = p.communicate()
        err = "\n".join(l for l in err.splitlines() if noise not in l)
        if p.returncode != 0:
            errs.append(f"hipcc failed ({p.returncode}): {' '.join(cmd[-3:])}\n{err}")
        elif verbose and err.strip():
            print(err, file=sys.stderr)
    if errs:
        raise RuntimeError("\n".join(errs))


def build(verbose: bool = True, extra=(), out: str = LIB) -> str:
    """Compiles every source to an object in parallel, links them, and
    replaces ``out`` atomically."""
    with tempfile.TemporaryDirectory(prefix="pa_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        _run([[hipcc(), *FLAGS, *extra, "-c", s, "-o", o] for s, o in zip(SOURCES, objs)], verbose)
        partial = out + ".tmp"
        _run([[hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", partial]], verbose)
        os.replace(partial, out)
    return out


if __name__ == "__main__":
    build()
