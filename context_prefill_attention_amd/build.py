"""Build libcpattn.so in-tree with hipcc for gfx950 only."""

from __future__ import annotations

import os
import subprocess
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libcpattn.so")
SOURCES = ["cp_meta.cpp", "cp_copy.hip", "cp_attn.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU instructions stay off: only scalar/float2 code is written
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every source into libcpattn.so (always recompiles)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(prefix=".libcpattn.", suffix=".so.tmp", dir=PKG_DIR)
    os.close(fd)
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    try:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
        if verbose:
            print(" ".join(cmd))
        os.replace(tmp, LIB_PATH)  # atomic: a process that already loaded the old file keeps it
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
