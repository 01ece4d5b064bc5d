"""Builds libgptq_hip.so from csrc/*.hip for gfx950 (hipcc cross-compiles,
no GPU needed).  Objects go to _build/ next to this file; the shared library
is written next to this file so the binding finds it in-tree."""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libgptq_hip.so")

ARCH = "gfx950"
HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # keep the compiler from forming packed fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE-rounded fp32 division: the grid fit and the encoder decide
    # integer codes from quotients
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wno-unused-command-line-argument",
]


# Per-file additions.  The matrix-core dequantizing product keeps its
# partial products in ordinary VGPRs (the fold into the result reads them
# every group; in the accumulation registers they would be copied out).
FILE_FLAGS: dict = {"k_dequant.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip (in parallel) and link the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    procs = []
    objs = []
    for src in srcs:
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        noise = [ln for ln in out.splitlines() if "not a recognized feature" not in ln]
        if p.returncode != 0:
            failed.append((src, "\n".join(noise)))
        elif verbose and noise:
            print("\n".join(noise))
    if failed:
        msg = "\n\n".join(f"{s}:\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
