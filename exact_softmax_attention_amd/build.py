"""Build libfa2.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

    python -m exact_softmax_attention_amd.build

The library lands next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SRCS = [os.path.join(PKG_DIR, "csrc", name) for name in ("fa2_fwd.hip", "fa2_bwd.hip", "fa2_merge.hip")]
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG_DIR, "libfa2.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # packed fp32 VALU ops stay off: hipcc would otherwise form v_pk_* from float code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}",
    ]


def build(verbose: bool = True, extra_flags: list[str] | None = None, out: str = LIB) -> str:
    """Compile the HIP sources into ``out`` (always recompiles). Returns the path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *compile_flags(), *(extra_flags or []), *SRCS, "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    noise = ("packed-fp32-ops", "not a recognized feature for this target")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
