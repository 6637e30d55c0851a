"""Build the gfx950 shared library libbitffn_moe.so in-tree.

    python -m bit_expert_ffn_top_amd.build

Every .hip file under csrc/ is compiled for gfx950 only (hipcc), then linked
into one shared library next to this file.  Packed-fp32 VALU instructions are
disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libbitffn_moe.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

CXXFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str, extra) -> str:
    cmd = [hipcc(), *CXXFLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stderr or "").splitlines() if ln.strip() and noise not in ln]
    return "\n".join(msgs)


def build(verbose: bool = False, extra_flags=None, jobs: int = 8) -> str:
    """Compile all sources and link the library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        futs = {ex.submit(_compile, s, o, extra): s for s, o in zip(srcs, objs)}
        for fut in cf.as_completed(futs):
            msg = fut.result()
            if verbose and msg:
                print(f"[{os.path.basename(futs[fut])}]\n{msg}", file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
