"""Build libteaf.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

    python -m tiled_exact_attention_forward_amd.build

Each source compiles to an object in _build/ (in parallel), then one shared library is
linked next to this file. Packed fp32 VALU instructions are disabled for device code.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libteaf.so")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd32.hip", "fa_decode.hip",
           "fa_merge.hip"]
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]
# The backward's dK/dV kernel pins its dK/dV accumulators to the AGPR file with inline
# MFMAs; the compiler's own MFMAs in that file (S, dP, dQ) then take VGPR destinations,
# so no accumulator moves between the two register files inside the loop.
EXTRA = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln]
    return obj, "\n".join(noise)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for obj, msg in results:
        if verbose and msg.strip():
            print(msg)
    tmp = LIB + ".tmp"
    cmd = ["hipcc", "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results],
           "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
