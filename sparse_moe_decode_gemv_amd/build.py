"""Build the HIP library in place: sparse_moe_decode_gemv_amd/libmoe_decode.so (gfx950).

Each source compiles to an object in parallel, then one link.  Always
recompiles.  Run as `python -m sparse_moe_decode_gemv_amd.build`; with
`--phase-trace`, the diagnostic variant libmoe_decode_phase.so instead, whose
single-launch layer kernel records phase timestamps (MOE_PHASE_TRACE).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_decode.so")
SOURCES = ["api.hip", "kernels_moe.hip", "kernels_lmhead.hip", "kernels_layer.hip", "kernels_layer_mxfp4.hip",
           "kernels_layer_nvfp4.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 arithmetic stays off on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


PHASE_LIB = os.path.join(HERE, "libmoe_decode_phase.so")


def _compile(src: str, obj_dir: str, extra: tuple) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    subprocess.check_call([HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj])
    return obj


def build(verbose: bool = False, phase_trace: bool = False) -> str:
    obj_dir = os.path.join(OBJ, "phase") if phase_trace else OBJ
    extra = ("-DMOE_PHASE_TRACE",) if phase_trace else ()
    lib = PHASE_LIB if phase_trace else LIB
    os.makedirs(obj_dir, exist_ok=True)
    if verbose:
        print(HIPCC, " ".join(FLAGS + list(extra)), "-c", SOURCES, flush=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, obj_dir, extra), SOURCES))
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", lib + ".tmp", *objs])
    os.replace(lib + ".tmp", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, phase_trace="--phase-trace" in sys.argv[1:])
    sys.exit(0)
