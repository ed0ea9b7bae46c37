"""Build libqlora_nf4.so for gfx950 with hipcc (in-tree, no JIT cache).

Usage: python -m bit_nf4_quantized_18_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqlora_nf4.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
# Packed-fp32 instructions are kept out of every device build; the quantizer
# and merge units are also built without floating-point contraction because
# their outputs (codes, scale codes, dequantized and merged values) are
# bit-exact.
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics"]
SOURCES = {
    "codebook.cpp": ["-ffp-contract=off"],
    "api.cpp": [],
    "quant_kernels.hip": DEVICE + ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt"],
    "merge_kernels.hip": DEVICE + ["-ffp-contract=off"],
    "lora_kernels.hip": DEVICE,
    "dropout_kernels.hip": DEVICE,
    "gemv_kernels.hip": DEVICE + ["-fhip-fp32-correctly-rounded-divide-sqrt"],
    "gemv_mfma.hip": DEVICE + ["-fhip-fp32-correctly-rounded-divide-sqrt"],
    "gemm_kernels.hip": DEVICE + ["-fhip-fp32-correctly-rounded-divide-sqrt"],
    "noalloc.hip": DEVICE,
}


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    return p.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src, flags in SOURCES.items():
        obj = os.path.join(BUILD, src.rsplit(".", 1)[0] + ".o")
        objs.append(obj)
        cmd = [HIPCC] + COMMON + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        msg = "\n".join(f"--- {s} ---\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    # -z defs: an unresolved symbol (a kernel stub the host pass did not emit,
    # say) fails the build here instead of the first dlopen
    rc, out = _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", "-o", tmp] + objs)
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
