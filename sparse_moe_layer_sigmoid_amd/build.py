"""Build libmoe.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m sparse_moe_layer_sigmoid_amd.build

Every ``csrc/*.hip`` file is compiled to an object with hipcc (in parallel), then linked
into ``sparse_moe_layer_sigmoid_amd/libmoe.so``.  The ceiling micro-benchmarks
(``ceilings/ceilings.hip``, measurement code driven by ``bench.py --ceilings``, not part of
the layer) go into their own ``libmoe_ceilings.so``.  Packed-FP32 instruction selection is
switched off for the device code (``-packed-fp32-ops``).
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libmoe.so")
CEILINGS_SRC = os.path.join(PKG, "ceilings", "ceilings.hip")
CEILINGS_LIB = os.path.join(PKG, "libmoe_ceilings.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-strict-aliasing",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({' '.join(cmd)}):\n{r.stdout}\n{r.stderr}")
    return r.stderr


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD_DIR, os.path.basename(s)[:-4] + ".o") for s in srcs]

    def compile_one(pair):
        s, o = pair
        return _run([HIPCC, *DEVICE_FLAGS, "-c", s, "-o", o])

    ceil_obj = os.path.join(BUILD_DIR, "ceilings.o")
    with ThreadPoolExecutor(jobs) as ex:
        logs = list(ex.map(compile_one, zip(srcs + [CEILINGS_SRC], objs + [ceil_obj])))
    for out, ins in ((LIB_PATH, objs), (CEILINGS_LIB, [ceil_obj])):
        tmp = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *ins])
        os.replace(tmp, out)
    if verbose:
        for s, log in zip(srcs + [CEILINGS_SRC], logs):
            if log.strip():
                print(f"--- {os.path.basename(s)}\n{log}", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
