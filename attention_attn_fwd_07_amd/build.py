"""Build the HIP library ``libattn_fwd.so`` in-tree for gfx950.

Sources: ``csrc/attn_fwd.hip`` (forward, split-KV, C ABI of include/attn_fwd.h)
and ``csrc/attn_bwd.hip`` (backward, include/attn_bwd.h), both including the
internal ``csrc/attn_common.h``.

Usage: ``python -m attention_attn_fwd_07_amd.build`` (or ``build()``).  The
library is compiled with hipcc, for gfx950 only, with packed-fp32 VALU ops
disabled (the compiler otherwise forms v_pk_* fp32 instructions by itself).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRCS = [os.path.join(PKG_DIR, "csrc", "attn_fwd.hip"),
        os.path.join(PKG_DIR, "csrc", "attn_bwd.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libattn_fwd.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattn_fwd.so")


def command(out: str = LIB) -> list[str]:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", *SRCS, "-o", out]


def build(verbose: bool = False) -> str:
    """Compile the library (always) and return its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        noise = "'-packed-fp32-ops' is not a recognized feature"
        msg = "\n".join(x for x in (res.stdout + res.stderr).splitlines() if noise not in x)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Return the library path, compiling it only if it does not exist yet."""
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
