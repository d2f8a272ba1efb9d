"""Build the HIP library ``libkvq.so`` for gfx950 with hipcc (in-tree, next to this file).

Each source is compiled to an object of its own, in parallel (the kernels of one file call no
device code of another), and the objects are linked into the shared library.
"""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvq.so")
OBJ = os.path.join(HERE, "_build")
# the HBM read-rate probe the benchmark reports beside the roofline, and the matrix-instruction
# accumulation probe of the FP8-math tests (neither is part of the cache's ABI)
PROBE_SRCS = [os.path.join(HERE, "probe", "read_probe.hip"), os.path.join(HERE, "probe", "mfma_probe.hip")]
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# gfx950 only.  Packed fp32 instructions are switched off for every kernel; fp32 division stays
# correctly rounded (hipcc's default) and denormals are not flushed (the append path relies on both).
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _link(srcs, out, verbose, extra_flags, jobs):
    os.makedirs(OBJ, exist_ok=True)
    stem = os.path.splitext(os.path.basename(out))[0]
    objs = [os.path.join(OBJ, f"{stem}.{os.path.splitext(os.path.basename(s))[0]}.o") for s in srcs]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *FLAGS, *extra_flags, "-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    _run([HIPCC, *FLAGS, *extra_flags, "-shared", *objs, "-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, extra_flags=(), jobs: int | None = None) -> str:
    jobs = jobs or min(8, os.cpu_count() or 1)
    _link(sources(), LIB, verbose, list(extra_flags), jobs)
    _link(PROBE_SRCS, PROBE_LIB, verbose, list(extra_flags), jobs)
    return LIB


# The host code (argument validation, sizing, the planning arithmetic) under clang's
# AddressSanitizer and UndefinedBehaviorSanitizer, linked to the shared sanitizer runtime; the
# device code is built as always.  The library goes to its own directory and is loaded in place of
# libkvq.so when KVQ_LIBRARY names it (tests/sanitize.py).
SAN_DIR = os.path.join(HERE, "_san")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g", "-shared-libsan"]


def build_sanitized(verbose: bool = False, jobs: int | None = None) -> str:
    global OBJ
    jobs = jobs or min(8, os.cpu_count() or 1)
    os.makedirs(SAN_DIR, exist_ok=True)
    out = os.path.join(SAN_DIR, "libkvq.so")
    saved, OBJ = OBJ, os.path.join(SAN_DIR, "obj")
    try:
        _link(sources(), out, verbose, SAN_FLAGS, jobs)
    finally:
        OBJ = saved
    return out


if __name__ == "__main__":
    print(build(verbose=True))
