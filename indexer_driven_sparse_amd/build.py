"""Build liblsa.so, the HIP C-ABI library, in-tree for gfx950.

Run ``python -m indexer_driven_sparse_amd.build`` (or ``__graft_entry__.build()``).
hipcc cross-compiles gfx950 device code on a host without a GPU.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed fp32 VALU ops stay off: plain fp32 code is used throughout
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the attention softmax
    # rescales O between products, which otherwise costs AGPR copies
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=1",
    "-I", INCLUDE,
    "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source (one object each, in parallel) and link them
    into indexer_driven_sparse_amd/liblsa.so. Every call compiles."""
    import concurrent.futures
    import tempfile

    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = jobs or min(len(sources()), os.cpu_count() or 1, 16)
    with tempfile.TemporaryDirectory(prefix="lsa_build_") as tmpdir:
        objs = []
        cmds = []
        for src in sources():
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            objs.append(obj)
            cmds.append([HIPCC, *compile_flags, "-c", src, "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            for cmd, rc in zip(cmds, pool.map(lambda c: subprocess.call(c), cmds)):
                if verbose or rc != 0:
                    print(" ".join(cmd), flush=True)
                if rc != 0:
                    raise subprocess.CalledProcessError(rc, cmd)
        tmp = LIB + ".tmp"
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.check_call(link)
        os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
