"""Build the gfx950 indexer library ``libmisa_indexer.so`` in-tree with hipcc.

    python -m long_context_sparse_05_amd.build_lib
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmisa_indexer.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH,
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep the compiler from emitting packed-fp32 VALU ops in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stderr or "").splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source to an object file (in parallel), then link the
    shared library; the objects go to a scratch folder that is removed."""
    import shutil
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    objdir = tempfile.mkdtemp(prefix="misa_build_")
    try:
        srcs = sources()
        objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
        compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
        jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(lambda so: _run([hipcc] + compile_flags + ["-c", so[0], "-o", so[1]], verbose),
                        zip(srcs, objs)))
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        os.replace(tmp, LIB)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
