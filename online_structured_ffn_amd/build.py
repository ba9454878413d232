"""Compile libpop.so for gfx950 with hipcc (in-tree, next to this file), and
its checking twin libpop_debug.so (POP_DEBUG: every entry point that takes
a partition's index lists validates them on the host first).

    python -m online_structured_ffn_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libpop.so")
OUT_DEBUG = os.path.join(PKG, "libpop_debug.so")
DEBUG_DEFINES = ("POP_DEBUG=1",)
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["pop_host.cpp", "trace.hip", "prefill.hip", "decode.hip", "prompt_ffn.hip", "moe.hip", "periodic.hip", "layer.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms stay off: every fp32 op is issued as a plain VOP
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src: str, defines=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, tag + os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    errs = [ln for ln in r.stderr.splitlines() if "warning" in ln and "packed-fp32-ops" not in ln]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    return obj


def build(verbose: bool = True, out: str = OUT, defines=()) -> str:
    """Compile and link the library; `defines` (NAME=VALUE strings) override
    the launch-shape tunables for a variant written to `out`."""
    os.makedirs(BUILD, exist_ok=True)
    tag = "" if not defines else f"v{abs(hash(tuple(defines))) % 10**8}_"
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, defines, tag), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def build_all(verbose: bool = True) -> None:
    build(verbose)
    build(verbose, OUT_DEBUG, DEBUG_DEFINES)


if __name__ == "__main__":
    build_all()
