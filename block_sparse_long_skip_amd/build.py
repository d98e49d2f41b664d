"""Build libblasst.so in-tree with hipcc for gfx950.

    python -m block_sparse_long_skip_amd.build [--jobs N]

Every HIP source under csrc/ is compiled for gfx950 only; the shared library
lands next to this file. Packed fp32 VALU instructions are disabled for every
device compilation.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libblasst.so")

SOURCES = ["api.cpp", "prefill_f32.hip", "prefill_bf16.hip", "backward_bf16.hip", "twopass.hip",
           "decode.hip", "decode_mla.hip"]
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source device flags. The latent-cache decode kernel keeps its output
# accumulators in VGPRs (MFMA VGPR form) because it rescales them on the VALU
# every time a running max grows; with the default AGPR form the compiler
# copies all of them between register files at every loop iteration.
# The two-pass map kernel reduces MFMA results with fmaxf: in the VGPR form and
# with NaNs excluded (no gap there can be NaN: both infinities are handled
# before any subtraction, and inputs must be finite) the reduction needs neither
# AGPR reads nor canonicalizing moves.
SOURCE_FLAGS = {"decode_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "twopass.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm is required to build libblasst)")
    return p


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ([hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS
           + SOURCE_FLAGS.get(src, []))
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(x for x in (r.stdout + r.stderr).splitlines() if noise not in x)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a symbol left undefined (for instance a kernel's launch stub the
    # host pass did not emit) fails the link here instead of the first dlopen
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(args.jobs, args.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())
