"""Build libbtq.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m bit_tensor_activation_amd.build [--asm DIR]

Flags that matter for the numerics:
  -ffp-contract=off  no implicit fused multiply-add. The moving average and
                     the quantizer's product must round as written. The
                     kernels write fma only where they mean it.
  no -ffast-math     fp32 division stays correctly rounded, denormals stay.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                     keeps the compiler from emitting packed fp32
                     instructions (v_pk_*_f32). This is a device flag; the
                     host pass warns that it does not know it.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbtq.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library needs ROCm's hipcc to build")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


OBJ_DIR = os.path.join(PKG, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into bit_tensor_activation_amd/libbtq.so.

    Each source compiles to an object of its own, in parallel (every kernel
    is launched from its own translation unit, so no device linking is
    needed), and the objects link into the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, os.path.basename(src).replace(".hip", ".o")) for src in srcs]
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(lambda so: _run([hipcc(), *COMMON_FLAGS, "-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


def device_asm(out_dir: str) -> list:
    """Write each source's gfx950 assembly to out_dir (for reading codegen).

    Returns the paths written. The sources compile in parallel."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        out = os.path.join(out_dir, os.path.basename(src).replace(".hip", ".s"))
        cmd = [hipcc(), *COMMON_FLAGS, "--cuda-device-only", "-S", src, "-o", out]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        return out

    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1, 8)) as ex:
        return list(ex.map(one, srcs))


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[1] == "--asm":
        device_asm(sys.argv[2])
    else:
        print(build(verbose=True))
