"""Build libcoli.so (the gfx950 HIP library) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcoli.so")
SOURCES = ["abi.hip", "gemv.hip", "mgemv.hip", "gemm.hip", "pgemm.hip", "dgemm.hip", "route.hip", "router.hip", "layer.hip", "mla.hip", "probe.hip"]
ARCH = os.environ.get("COLI_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-rdc", "-Wall", "-Wno-unused-function",
]


# Extra compiler options per source (none at present).
OWN_FLAGS: dict = {}


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link libcoli.so."""
    import concurrent.futures
    import tempfile
    with tempfile.TemporaryDirectory(prefix="coli_build_") as tmpd:
        jobs = []
        for name in SOURCES:
            obj = os.path.join(tmpd, name + ".o")
            cmd = ["hipcc", *[f for f in FLAGS if f != "-shared"], *OWN_FLAGS.get(name, []), "-c",
                   os.path.join(CSRC, name), "-o", obj]
            jobs.append((cmd, obj))
        if verbose:
            for cmd, _ in jobs:
                print(" ".join(cmd), flush=True)
        workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            for r in ex.map(lambda j: subprocess.run(j[0]), jobs):
                if r.returncode != 0:
                    raise subprocess.CalledProcessError(r.returncode, r.args)
        tmp = LIB + ".tmp"
        cmd = ["hipcc", "-fPIC", "-shared", f"--offload-arch={ARCH}", *[o for _, o in jobs], "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
