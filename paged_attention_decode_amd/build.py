"""Build libpagedattn.so in-tree with hipcc for gfx950.

``python -m paged_attention_decode_amd.build`` or ``build()`` from Python.
Sources are compiled in parallel to objects under ``_build/`` and linked
into ``paged_attention_decode_amd/libpagedattn.so``; the benchmark's
streaming-read kernel goes into its own ``libpa_stream_read.so``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = PKG / "_build"
LIB = PKG / "libpagedattn.so"
SOURCES = ["api.hip", "decode.hip", "prefill.hip", "store_kvcache.hip", "block_manager.cpp"]
# Measurement-only library of the benchmark (streaming-read ceiling); not part of libpagedattn.
STREAM_SOURCE = "stream_read.hip"
STREAM_LIB = PKG / "libpa_stream_read.so"
ARCH = os.environ.get("PA_OFFLOAD_ARCH", "gfx950")

# Packed fp32 instructions are kept out of the generated code. Matrix-core results stay in
# ordinary VGPRs (no accumulator-register copies around the online-softmax rescale).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-I", str(INCLUDE), "-I", str(CSRC)]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and Path(cand).exists():
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)


def build(verbose: bool = False, extra_flags=()) -> Path:
    hipcc = _hipcc()
    BUILD.mkdir(exist_ok=True)
    srcs = SOURCES + [STREAM_SOURCE]
    objs = [BUILD / (Path(s).stem + ".o") for s in srcs]
    cmds = [[hipcc, *COMMON, *extra_flags, "-c", str(CSRC / s), "-o", str(o)] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    for lib, lib_objs in ((LIB, objs[:-1]), (STREAM_LIB, objs[-1:])):
        tmp = lib.with_suffix(".so.tmp")
        _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *map(str, lib_objs), "-o", str(tmp)], verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    out = build(verbose="-v" in sys.argv)
    print(f"built {out}")
