"""Builds libpsw.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m paged_sliding_window_page_amd.build

Each translation unit is compiled to an object under ``_build/`` in parallel and
then linked into ``paged_sliding_window_page_amd/libpsw.so``.  Every call
recompiles.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpsw.so")

SOURCES = ["psw_host.cpp", "psw_kv.cpp", "psw_entry.hip", "psw_attn256.hip", "psw_attn512.hip",
           "psw_prep.hip", "psw_decode.hip", "psw_clock.hip", "psw_noalloc.hip",
           "psw_prefill512.hip"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}",
        "--offload-arch=gfx950",
        # no packed fp32 instructions anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


# Per-file code-generation options.  The head_dim-256 attention kernels keep
# their MFMA accumulators (O and S) in VGPRs so the softmax and the rare O
# rescale touch them without AGPR round trips; Q fragments then go to AGPRs,
# which the MFMA reads directly.  (At head_dim 512, O alone fills 256
# registers, so it stays in AGPRs.)
EXTRA = {"psw_attn256.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "psw_attn512.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        # host-only translation unit: no device code
        cmd = [_hipcc(), "-O2", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
               "-x", "c++", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libpsw.so failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
