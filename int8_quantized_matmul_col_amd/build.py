"""Builds libint8mm.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m int8_quantized_matmul_col_amd.build

Each source is compiled to an object under ``_build/`` (in parallel), then
linked into ``int8_quantized_matmul_col_amd/libint8mm.so``.  The measurement
probes (``csrc/ceilings.hip``) become a library of their own,
``libint8mm_ceilings.so``, which only the benchmark loads.  Flags:

* ``--offload-arch=gfx950`` only (MI355X).
* No fast-math: the quantizer relies on IEEE-correctly-rounded fp32 division.
* ``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the compiler
  from forming packed fp32 instructions.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libint8mm.so")
PROBE_LIB_PATH = os.path.join(HERE, "libint8mm_ceilings.so")
PROBE_SOURCES = ["ceilings.hip"]

SOURCES = ["api.hip", "prepare.hip", "activation.hip", "gemm_prefill.hip", "gemm_decode.hip"]
HEADERS = ["device_common.h", "launch.h"]

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libint8mm.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature; drop that line
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


def _link(objs, path: str, verbose: bool) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    """Compiles every source, links libint8mm.so and the probe library;
    returns the path of libint8mm.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB_PATH, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
