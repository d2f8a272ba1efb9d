"""Build the HIP library ``libkvq.so`` for gfx950 with hipcc (in-tree, next to this file)."""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvq.so")
# the HBM read-rate probe the benchmark reports beside the roofline (not part of the cache's ABI)
PROBE_SRC = os.path.join(HERE, "probe", "read_probe.hip")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# gfx950 only.  Packed fp32 instructions are switched off for every kernel; fp32 division stays
# correctly rounded (hipcc's default) and denormals are not flushed (the append path relies on both).
FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=()) -> str:
    for srcs, out in ((sources(), LIB), ([PROBE_SRC], PROBE_LIB)):
        cmd = [HIPCC, *FLAGS, *extra_flags, *srcs, "-o", out + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
