"""Build libmcs.so (the C-ABI library of the hot path) for gfx950 with hipcc.

Usage: python -m sparse_attention_diffusion_attn_amd.build [--sanitized]
Objects go to <package>/_build/, the library to <package>/libmcs.so.

--sanitized also builds <package>/_build/libmcs_san.so: the same library with
its host code (mcs_api.cpp: argument validation, layout and workspace
arithmetic, launch set-up) compiled by the host compiler under
AddressSanitizer and UndefinedBehaviorSanitizer, linked with the unchanged
kernel objects.  Only host code is instrumented.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmcs.so")
SOURCES = ["attn.hip", "select.hip", "pddp.hip", "blocks.hip", "kmeans.hip", "noalloc.hip", "mcs_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no accvgpr moves around the softmax)
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")


def build(verbose: bool = False) -> str:
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        list(ex.map(_compile, SOURCES, objs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


SAN_OUT = os.path.join(PKG, "_build", "libmcs_san.so")
GXX = os.environ.get("CXX_HOST", "g++")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def build_sanitized(verbose: bool = False) -> str:
    """libmcs_san.so: mcs_api.cpp under ASan + UBSan (host compiler), the
    kernel objects of the last build() unchanged."""
    bdir = os.path.join(PKG, "_build")
    kernel_objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(verbose)
    api_obj = os.path.join(bdir, "mcs_api_san.o")
    cmd = [GXX, "-std=c++17", "-O1", "-g", "-fPIC", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-c", os.path.join(CSRC, "mcs_api.cpp"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"host compile of mcs_api.cpp failed:\n{r.stderr}")
    cmd = [GXX, "-shared", *SAN_FLAGS, "-o", SAN_OUT, api_obj, *kernel_objs,
           "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the sanitized library failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    build(verbose=True)
    if "--sanitized" in sys.argv[1:]:
        build_sanitized(verbose=True)
    sys.exit(0)
