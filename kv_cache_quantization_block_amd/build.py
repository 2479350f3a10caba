"""Build libtq.so (the C-ABI library with the gfx950 kernels) in place.

    python -m kv_cache_quantization_block_amd.build

hipcc cross-compiles for gfx950 without a GPU.  Packed-fp32 instructions are
disabled for the device code (the host pass warns that it does not know the
feature; that warning is harmless).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libtq.so")
SOURCES = [os.path.join(CSRC, f) for f in ("kernels.hip", "codebook.cpp", "api.cpp")]
HEADERS = [os.path.join(CSRC, "internal.h"), os.path.join(ROOT, "include", "tq.h")]
# sha256 of the sources a library was built from, written beside it at build time and
# checked by the binding before it loads the library
SRC_SHA = LIB + ".srcsha"


def source_sha() -> str:
    """sha256 over the bytes of every source and header libtq.so is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in SOURCES + HEADERS:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libtq.so)")


def command(out: str = LIB, extra: list[str] | None = None) -> list[str]:
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", out,
            *SOURCES, *(extra or [])]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    sha = source_sha()
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    with open(SRC_SHA, "w") as fh:
        fh.write(sha + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
