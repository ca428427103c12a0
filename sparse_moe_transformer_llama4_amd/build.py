"""Build libmoe355.so (the C-ABI library) from csrc/*.hip for gfx950 with hipcc.

Usage: python -m sparse_moe_transformer_llama4_amd.build [--debug]   (or build() from Python)
The library lands in sparse_moe_transformer_llama4_amd/_lib/ (in-tree); with
--debug (build(debug=True)) the same sources compiled with -DMOE_DEBUG land in
_lib/libmoe355_debug.so: device-side checks of the routing and of every GEMM
tile, reported as MOE_ERR_CHECK (include/moe.h, moe_debug_flags).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libmoe355.so")
DEBUG_LIB = os.path.join(LIBDIR, "libmoe355_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-unit code generation.  The 64- and 128-row bf16 GEMM tiles, the
# weight-streaming decode kernels, the router partials and the fp32 MFMA
# GEMMs keep their accumulators in VGPRs (VGPR-form MFMAs): with the AGPR form
# the register allocator copied them between registers, and in the decode
# kernels parked other values in AGPRs, inside the main loops.  The 256-row
# tiles need both register files (with the VGPR form they spill).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
UNIT_FLAGS = {
    "gemm_bf16.hip": _VGPR_FORM,
    "gemm_decode.hip": _VGPR_FORM,
    "route.hip": _VGPR_FORM,
    "gemm.hip": _VGPR_FORM,
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, objdir: str, extra) -> str:
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *UNIT_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=(), debug: bool = False) -> str:
    objdir = os.path.join(LIBDIR, "obj_debug" if debug else "obj")
    lib = DEBUG_LIB if debug else LIB
    extra = list(extra) + (["-DMOE_DEBUG"] if debug else [])
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    args = sys.argv[1:]
    build(verbose=True, extra=[a for a in args if a != "--debug"], debug="--debug" in args)
