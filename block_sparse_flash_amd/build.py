"""Build ``libsplash.so`` (the C-ABI library with the gfx950 kernels) in-tree.

Every source under ``csrc/`` is compiled with hipcc for gfx950 only and
linked into ``block_sparse_flash_amd/libsplash.so``.  Run as
``python -m block_sparse_flash_amd.build``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsplash.so")

SOURCES = [
    "errors.cpp",
    "mask_compile.cpp",
    "splash_api.cpp",
    "splash_fwd_f32.hip",
    "splash_fwd_bf16.hip",
    "splash_fwd_bf16_d192.hip",
    "splash_fwd_bf16_d64.hip",
    "splash_split_merge.hip",
    "splash_bwd_api.cpp",
    "splash_bwd_bf16.hip",
    "splash_noalloc.hip",
    "clock_probe.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libsplash")
    return path


def common_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        f"-I{INCLUDE}", f"-I{CSRC}",
        # Packed fp32 VALU instructions stay disabled on the device.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
    ]


# Per-source extra flags.  The bf16 kernel never produces NaN inside the
# softmax (masked scores are -inf, all other values finite), so it is built
# without IEEE NaN canonicalisation: fmaxf becomes a bare v_max3_f32.
_FWD_FLAGS = ["-fno-honor-nans", "-mno-amdgpu-ieee"]
EXTRA_FLAGS = {
    "splash_fwd_bf16.hip": _FWD_FLAGS,
    "splash_fwd_bf16_d192.hip": _FWD_FLAGS,
    "splash_fwd_bf16_d64.hip": _FWD_FLAGS,
}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *common_flags(), *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip() and verbose:
        print(msg, file=sys.stderr)
    return obj


def build_library(verbose: bool = False) -> str:
    """Compile every source and link ``libsplash.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
