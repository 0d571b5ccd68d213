"""Builds libpv_tower.so in-tree with hipcc for gfx950.

Usage: ``python -m vlm_vision_encoder_amd.build_lib`` (or
``__graft_entry__.build()``).  Objects go to ``vlm_vision_encoder_amd/_build``;
the library lands next to this file.  Always recompiles.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpv_tower.so")

SOURCES = ["plan.cpp", "tower.cpp", "embcache.cpp", "maps.hip", "norm.hip", "prep.hip", "gemm_bf16.hip",
           "attn_bf16.hip", "f32_path.hip", "scatter.hip", "hash.hip"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
# packed fp32 VALU instructions are kept out of every device code object
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the tower library)")


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + COMMON + DEVICE + ["-D" + d for d in defines]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if err:
        sys.stderr.write(err + "\n")
    return obj


PROBE_SRC = "probe_issue.hip"
PROBE = os.path.join(PKG, "probe_issue")


def build_probe(verbose: bool = True) -> str:
    """Builds the MFMA / VALU overlap microbenchmark (an executable, not part
    of the library)."""
    cmd = [hipcc()] + COMMON + DEVICE + [os.path.join(CSRC, PROBE_SRC), "-o", PROBE + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"probe build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(PROBE + ".tmp", PROBE)
    if verbose:
        print(f"built {PROBE}")
    return PROBE


def build(verbose: bool = True, jobs: int = 8, out: str = LIB, build_dir: str = BUILD, defines=()) -> str:
    """Compiles all sources (optionally with extra -D defines) and links `out`."""
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()
