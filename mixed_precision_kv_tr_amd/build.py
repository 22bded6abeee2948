"""Builds libtriroute.so (C ABI + gfx950 kernels) in-tree with hipcc.

    python -m mixed_precision_kv_tr_amd.build        # or __graft_entry__.build()

Flags: gfx950 only, -O3, no fast-math (the quantizer's divides must stay correctly rounded and
fp32 denormals must be kept), packed-FP32 instruction selection disabled.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtriroute.so")
SOURCES = ["cache.cpp.hip", "decode.cpp.hip", "prefill.cpp.hip", "controller.cpp.hip", "moe.cpp.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose: bool = False) -> str:
    cc = hipcc()
    objs = []
    tmp = os.path.join(PKG, "_build")
    os.makedirs(tmp, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmp, src.replace(".cpp.hip", ".o"))
        cmd = [cc, *flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if verbose and errs.strip():
            print(errs)
        objs.append(obj)
    tmp_lib = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp_lib, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp_lib, LIB)
    _record_revision(tmp)
    return LIB


def _record_revision(build_dir: str) -> None:
    """Writes the git commit the library was built from (with "+dirty" if the tree had changes)
    next to the objects, so that a copy of the tree without .git still names it."""
    try:
        head = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
    except (OSError, subprocess.SubprocessError):
        return
    if head.returncode != 0 or not head.stdout.strip():
        return
    rev = head.stdout.strip() + ("+dirty" if dirty.returncode == 0 and dirty.stdout.strip() else "")
    with open(os.path.join(build_dir, "REVISION"), "w") as f:
        f.write(rev + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
