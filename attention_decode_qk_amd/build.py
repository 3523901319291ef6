"""Build the gfx950 C-ABI library libmi355x_gated_attn.so in-tree with hipcc.

    python -m attention_decode_qk_amd.build [--force]

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops) and MFMA results
kept in ordinary VGPRs (-mllvm -amdgpu-mfma-vgpr-form: the scores and
accumulators are read and rescaled by vector ALU code, which otherwise pays a
move out of the accumulation registers for every value), then linked into one
shared library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmi355x_gated_attn.so")
# The host-sanitized build (address + undefined behaviour in the host code
# only; the gfx950 code is unchanged): its own objects and library, loaded in
# place of the product library when MI355X_GA_LIB names it.
SAN_OUT_DIR = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(HERE, "libmi355x_gated_attn_san.so")
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]
SOURCES = ["step_kernel.hip", "extend_kernel.hip", "meta_kernel.hip", "qk_norm_kernel.hip", "api.cpp"]
HEADERS = [os.path.join(CSRC, "kernels.h"), os.path.join(CSRC, "numerics.h"),
           os.path.join(CSRC, "step_device.h"),
           os.path.join(os.path.dirname(HERE), "include", "mi355x_gated_attn.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-result"]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_OUT_DIR if sanitize else OUT_DIR, os.path.splitext(src)[0] + ".o")
    flags = FLAGS + (SAN_FLAGS if sanitize else [])
    cmd = [HIPCC, *flags, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(force: bool = True, verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source and link the library (sanitize=True: the
    host-sanitized one); returns its path."""
    out_dir, lib = (SAN_OUT_DIR, SAN_LIB) if sanitize else (OUT_DIR, LIB)
    os.makedirs(out_dir, exist_ok=True)
    if not force and os.path.exists(lib):
        newest = max(os.path.getmtime(os.path.join(CSRC, s)) for s in SOURCES)
        newest = max([newest] + [os.path.getmtime(h) for h in HEADERS])
        if os.path.getmtime(lib) >= newest:
            return lib
    with ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = lib + ".tmp"
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-shared-libsan"] if sanitize else []
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(force="--force" in sys.argv or True, verbose=True)
