"""Build libmla.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Usage: python -m mla_latent_kv_34_amd.build   (or build() from Python)
Every source under csrc/ is compiled by hipcc into _build/, then linked into
mla_latent_kv_34_amd/libmla.so.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmla.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "append.hip", "generic.hip", "decode_v2.hip", "prefill_v2.hip", "proj.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


GENERATED = [("gen_splitkv_asm.py", "splitkv_asm.h"), ("gen_prefill_asm.py", "prefill_asm.h")]


def _generate() -> None:
    """Regenerate the inline-assembly headers of the MFMA kernels."""
    for script, header in GENERATED:
        gen = os.path.join(CSRC, script)
        r = subprocess.run([sys.executable, gen], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{gen} failed:\n{r.stderr}")
        out = os.path.join(CSRC, header)
        old = open(out).read() if os.path.exists(out) else None
        if old != r.stdout:
            with open(out, "w") as f:
                f.write(r.stdout)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _generate()
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
