"""Compile libsva.so (hand-written HIP for gfx950) in place.

Each .hip source is compiled to an object under _build/ in parallel and then
linked into ``sparse_attention_long_head_amd/libsva.so``.  Always recompiles.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsva.so")
SOURCES = ["sva_api.hip", "attention.hip", "kmeans.hip", "permute.hip", "select.hip", "radial.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # No packed fp32 VALU forms (v_pk_add/mul/fma_f32) in any kernel.  The
    # feature switch acts on the device pass; the host (x86) pass does not know
    # it and prints a harmless "not a recognized feature" warning.  The switch
    # cannot be scoped to the device pass alone (-Xarch_device takes no option
    # with an argument), so check_device_code() verifies the result instead.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
LLVM = "/opt/rocm/llvm/bin"
PACKED_FP32 = re.compile(r"\bv_pk_(add|mul|fma)_f32\b")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsva)")


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def check_device_code(obj: str) -> int:
    """Disassemble the gfx950 code object inside ``obj`` and raise if it holds a
    packed fp32 VALU instruction; returns the number of instructions read."""
    fat, co = obj + ".fatbin", obj + ".co"
    r = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "-S", obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"llvm-readelf failed on {obj}:\n{r.stderr}")
    if ".hip_fatbin" not in r.stdout:
        return 0                     # host code only (no kernels in this source)
    steps = [[os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj,
              os.devnull],
             [os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
              f"--input={fat}", f"--targets=hipv4-amdgcn-amd-amdhsa--{ARCH}", f"--output={co}"]]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"device code check of {obj} failed:\n{r.stderr}")
    r = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", co], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"llvm-objdump failed on {co}:\n{r.stderr}")
    bad = [ln.strip() for ln in r.stdout.splitlines() if PACKED_FP32.search(ln)]
    if bad:
        raise RuntimeError(f"{os.path.basename(obj)}: packed fp32 VALU instructions in the "
                           f"device code ({len(bad)}), e.g. {bad[0]}")
    return sum(1 for ln in r.stdout.splitlines() if ln.startswith("\t"))


def build(extra_flags=(), jobs: int = 5) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
        list(ex.map(check_device_code, objs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
