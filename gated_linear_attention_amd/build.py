"""Build libsgla.so in-tree for gfx950.

Every HIP source is compiled with hipcc for gfx950 only; the host API is
compiled by hipcc as well.  The shared library is linked against the HIP
runtime that PyTorch loads (torch/lib/libamdhip64.so) when torch is present,
so that a process using torch for device memory and streams has exactly one
HIP runtime and torch's stream handles are valid in libsgla.  Without torch
the ROCm installation's runtime is used.

Usage: python gated_linear_attention_amd/build.py   (or build() from Python).  Run it
as a script: importing the package loads the library that is already built.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "sgla")
LIB_PATH = os.path.join(PKG, "libsgla.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-command-line-argument",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; libsgla needs ROCm's hipcc to build")


def hip_runtime_dir() -> str:
    """Directory of the libamdhip64.so the library links against."""
    try:
        import torch  # noqa: F401
        d = os.path.join(os.path.dirname(torch.__file__), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    except Exception:
        pass
    return "/opt/rocm/lib"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc()] + HIPCC_FLAGS + list(extra) + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra_flags=(), out_path: str = LIB_PATH) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags), srcs))
    rt = hip_runtime_dir()
    tmp = out_path + ".tmp"
    cmd = ["g++", "-shared", "-o", tmp] + objs + [
        f"-L{rt}", "-l:libamdhip64.so", f"-Wl,-rpath,{rt}", "-Wl,--no-undefined", "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out_path)
    if verbose:
        print(f"built {out_path} (HIP runtime from {rt})")
    return out_path


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
