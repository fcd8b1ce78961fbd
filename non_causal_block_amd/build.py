"""Build libdflash_attn.so (gfx950) in-tree with hipcc.

    python -m non_causal_block_amd.build [--verbose] [--timeline]

Each csrc/*.hip is compiled to an object under _build/ (in parallel), then
linked into non_causal_block_amd/libdflash_attn.so.  --timeline builds the same
sources with -DDFLASH_TIMELINE (objects under _build/timeline/) into
libdflash_attn_timeline.so, whose attention kernel also writes per-workgroup
wall-clock stamps (dflash_timeline_set_buffer; `bench.py --timeline`).  Every HIP compile line
turns off the packed-fp32 target feature (``-packed-fp32-ops``): ordinary
float code must not be lowered to v_pk_* fp32 instructions on this target.
"""
from __future__ import annotations

import argparse
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdflash_attn.so")
TIMELINE_LIB = os.path.join(PKG, "libdflash_attn_timeline.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str, verbose: bool, outdir: str = BUILD, defines=()) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr).strip()
    # hipcc's host pass does not know the gfx feature; that one line is noise
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n" + "\n".join(lines))
    if lines and verbose:
        print("\n".join(lines), flush=True)
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    outdir = os.path.join(BUILD, "timeline") if timeline else BUILD
    lib = TIMELINE_LIB if timeline else LIB
    defines = ("DFLASH_TIMELINE",) if timeline else ()
    os.makedirs(outdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, outdir, defines), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed\n" + r.stdout + r.stderr)
    os.replace(tmp, lib)
    return lib


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--timeline", action="store_true", help="the timeline build (libdflash_attn_timeline.so)")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose, timeline=args.timeline))
    return 0


if __name__ == "__main__":
    sys.exit(main())
