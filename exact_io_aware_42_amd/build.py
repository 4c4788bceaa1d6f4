"""Build libfa2.so in-tree with hipcc for gfx950.

    python -m exact_io_aware_42_amd.build [--all]

Compiles the HIP kernels and the C ABI into exact_io_aware_42_amd/libfa2.so (with --all also
libfa2_debug_sync.so, the race-check build). Packed-fp32
VALU instructions are disabled for all device code.
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libfa2.so")
# the same sources with an extra wait and workgroup barrier at every LDS stage hand-over
# (FA2_DEBUG_SYNC); its outputs must equal libfa2.so's bit for bit (a race check)
DEBUG_SYNC_LIB_PATH = os.path.join(PKG_DIR, "libfa2_debug_sync.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["fa2_api.cpp", "fa2_fwd.hip", "fa2_bwd.hip"]
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # NaNs are not produced on purpose anywhere in the kernels; without this flag every fmaxf on
    # an MFMA result is preceded by a canonicalising v_max_f32
    "-fno-honor-nans",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: softmax reads the score accumulators with plain VALU ops, so
    # AGPR-form MFMAs would need a v_accvgpr_read per element
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # the ILP-oriented machine scheduler issues LDS operand reads well ahead of the MFMAs that
    # consume them (the default occupancy-oriented one waits on each read right before its MFMA)
    "-mllvm", "-amdgpu-sched-strategy=iterative-ilp",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def build(verbose: bool = False, extra_flags=None, out_path: str = LIB_PATH) -> str:
    """Compile every source and link libfa2.so (or `out_path`); returns its path. Raises on
    failure."""
    objs = []
    tmp_dir = os.path.join(PKG_DIR, "_build", hashlib.sha1(out_path.encode()).hexdigest()[:8])
    os.makedirs(tmp_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(tmp_dir, src + ".o")
        cmd = [HIPCC, *COMMON_FLAGS, *(extra_flags or []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the packed-fp32 feature and says so: harmless
        noise = "not a recognized feature for this target"
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        objs.append(obj)
    tmp_lib = out_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp_lib, out_path)
    return out_path


def build_all(verbose: bool = False):
    """libfa2.so and its FA2_DEBUG_SYNC twin; returns both paths."""
    return (build(verbose=verbose),
            build(verbose=verbose, extra_flags=["-DFA2_DEBUG_SYNC"],
                  out_path=DEBUG_SYNC_LIB_PATH))


if __name__ == "__main__":
    if "--all" in sys.argv:
        print(*build_all(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
