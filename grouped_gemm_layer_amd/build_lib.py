"""Build the HIP library of the MoE layer for gfx950 (cross-compiles without a GPU).

    python -m grouped_gemm_layer_amd.build_lib        # or build() below
    python -m grouped_gemm_layer_amd.build_lib -D MOE_CFG_ROW_FWD=256,256,2,4,2,2,64,4,1

Produces grouped_gemm_layer_amd/libmoe_gfx950.so from csrc/*.hip.  `-D NAME=VALUE`
overrides one of the sources' compile-time settings (tile shapes, work-list
order and chunk size: the `#ifndef MOE_...` blocks); `--out PATH` writes the
library elsewhere.  Variants build their objects in a directory of their own.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_gfx950.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["route.hip", "router.hip", "combine.hip", "gemm_bf16.hip", "gemm_fp32.hip", "mxfp8.hip", "gemm_mx8.hip", "api.hip"]

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
]


def _compile(src: str, verbose: bool, defines=(), objdir: str = BUILD) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *("-D" + d for d in defines), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out)
    return obj


def build_library(verbose: bool = False, defines=(), out: str | None = None) -> str:
    defines = tuple(defines)
    for d in defines:
        if not d.startswith("MOE_"):
            raise ValueError(f"not a setting of the sources: {d}")
    objdir = BUILD if not defines else os.path.join(
        BUILD, "v_" + hashlib.sha1(" ".join(defines).encode()).hexdigest()[:12])
    os.makedirs(objdir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, defines, objdir), SOURCES))
    out = out or os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print("built", out, flush=True)
    return out


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build the gfx950 library of the MoE layer")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="NAME=VALUE")
    ap.add_argument("--out", default=None)
    ap.add_argument("-q", action="store_true")
    args = ap.parse_args()
    build_library(verbose=not args.q, defines=args.defines, out=args.out)
