"""Build the CPU oracle's shared library (plain C, gcc).

TEST INFRASTRUCTURE ONLY: the oracle is loaded by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "libkvq_oracle.so")

# -ffp-contract=off: no fused multiply-add may change a rounding the definitions fix;
# no -ffast-math: IEEE semantics, NaN / inf / signed zero and nearbyint() ties-to-even hold.
CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared"]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


# The same source under clang's AddressSanitizer and UndefinedBehaviorSanitizer (the shared
# runtime, so that one runtime serves this library and the HIP library's sanitized build in one
# process).  Loaded in place of libkvq_oracle.so when KVQ_ORACLE_LIBRARY names it.
CLANG = os.environ.get("KVQ_SAN_CC", "/opt/rocm/llvm/bin/clang")
SAN_LIB = os.path.join(HERE, "_san", "libkvq_oracle.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-g", "-shared-libsan"]


def build_sanitized(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    flags = [f for f in CFLAGS if f != "-O2"] + ["-O1"]
    cmd = [CLANG, *flags, *SAN_FLAGS, SRC, "-o", SAN_LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SAN_LIB + ".tmp", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    print(build(verbose=True))
