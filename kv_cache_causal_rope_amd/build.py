"""Build libkvrope.so (the C-ABI library with the gfx950 attention kernels,
include/kvrope.h) and libkvrope_probes.so (the benchmark's measurement helpers,
include/kvrope_probes.h).

    python -m kv_cache_causal_rope_amd.build

Compiles every ``csrc/*.hip`` with hipcc for gfx950 into the package directory.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libkvrope.so")
PROBES_LIB = os.path.join(HERE, "libkvrope_probes.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = os.environ.get("KVROPE_ARCH", "gfx950")

SOURCES = ["api.hip", "rope_append.hip", "prefill.hip", "decode.hip", "gemm.hip"]
PROBE_SOURCES = ["probes.hip"]

# Packed fp32 instructions are switched off for all device code (the compiler would
# otherwise form v_pk_* from ordinary float code).
HIPFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in [os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")]:
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIPFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    subprocess.run([hipcc(), "-shared", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBES_LIB)
    if verbose:
        print(LIB)
        print(PROBES_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
