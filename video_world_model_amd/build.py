"""Build the QuantWM HIP library (libqwm.so) in-tree for gfx950.

Usage: python -m video_world_model_amd.build  (or call build()).

Flags that the bit-exact quantizer depends on:
  -ffp-contract=off                          no fused multiply-add is formed
  -fhip-fp32-correctly-rounded-divide-sqrt   float '/' is IEEE correctly rounded
  -fno-gpu-flush-denormals-to-zero           subnormals are kept
and -Xclang -target-feature -Xclang -packed-fp32-ops keeps the compiler from
emitting packed float32 VALU instructions.
"""

from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqwm.so")
ARCH = os.environ.get("QWM_OFFLOAD_ARCH", "gfx950")

SOURCES = ["qwm_host.hip", "kern_quant.hip", "kern_calib.hip", "kern_attend.hip", "kern_attend_bf16.hip",
           "kern_decode.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def source_files():
    """Every file the library is compiled from, as (path relative to the repo, absolute path)."""
    files = [("include/qwm.h", os.path.join(INCLUDE, "qwm.h"))]
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            files.append((f"video_world_model_amd/csrc/{f}", os.path.join(CSRC, f)))
    return files


def source_hash() -> str:
    """First 16 hex digits of a SHA-256 over the library's sources (name and
    bytes of each file, in name order). The build stamps it into
    qwm_version(), so a loaded library can be matched against the tree."""
    h = hashlib.sha256()
    for rel, path in source_files():
        h.update(rel.encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libqwm.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    stamp = f'-DQWM_SOURCE_HASH="{source_hash()}"'
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *CFLAGS, stamp, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = min(len(cmds), int(os.environ.get("MAX_JOBS", "4")) or 1)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
