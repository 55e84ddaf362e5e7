"""Compiles the gfx950 HIP libraries in-tree with hipcc: libmxfp8.so (the
casts and their consumer, behind include/mxfp8.h) and libmxstream.so (the
streaming bandwidth probe behind include/mxstream.h, measurement only)."""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libmxfp8.so")
SOURCES = [os.path.join(CSRC, "mxfp8.hip")]
STREAM_LIB_PATH = os.path.join(PKG_DIR, "libmxstream.so")
STREAM_SOURCES = [os.path.join(CSRC, "mx_stream.hip")]
ARCH = "gfx950"


def kernel_source_hash() -> str:
    """Short hash of the kernel sources (the .hip/.hpp/.h files under
    csrc/): ties a recorded profile to the code it measured."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if not name.endswith((".hip", ".hpp", ".h")):
            continue
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxfp8.so)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        # keep fp32 math scalar: no packed-fp32 instructions are generated
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def build(out: str = LIB_PATH, extra_flags: list[str] | None = None, verbose: bool = False,
          sources: list[str] | None = None) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *compile_flags(), *(extra_flags or []), "-shared", "-o", tmp, *(sources or SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "'-packed-fp32-ops' is not a recognized feature"
    text = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{text}")
    if verbose and text.strip():
        print(text, flush=True)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> None:
    build(verbose=verbose)
    build(STREAM_LIB_PATH, verbose=verbose, sources=STREAM_SOURCES)


if __name__ == "__main__":
    build_all(verbose=True)
