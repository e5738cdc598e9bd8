"""Build libssattn.so (the C-ABI library with its gfx950 kernels) in-tree.

Usage: ``python -m block_sparse_attention_online_amd.build`` (or call
``build()``).  Compiles every source under ``csrc/`` with hipcc for gfx950
into ``_build/`` and links the shared library next to this file.  Always
recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssattn.so")
ARCH = "gfx950"

# Packed fp32 instructions are kept out of every device build.  MFMA results
# stay in VGPRs (the MFMA's VGPR form): the score accumulators feed vector ALU
# work (max, exp), and in AGPRs every such use costs a v_accvgpr_read and
# every rescale a read and a write.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
# ... except where the accumulators alone fill the 256 architectural VGPRs:
# the latent decode keeps a [512 x 32] fp32 output block per wave in the
# accumulation registers, the backward's dK/dV kernel the dK^T and dV^T
# blocks of 32 keys.
AGPR_FORM = {"decode_mla.hip", "prefill_bwd_dkdv.hip"}
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    flags = DEVICE_FLAGS
    if os.path.basename(src) in AGPR_FORM:
        flags = [f for f in DEVICE_FLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
    cmd = [hipcc(), *COMMON, *flags, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), *COMMON, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in r.stderr.splitlines() if noise not in ln)
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
