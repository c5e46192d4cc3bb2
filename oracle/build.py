"""Builds the CPU oracle (test infrastructure) into oracle/liboracle.so with gcc.

The flags keep every float32 step of the quantizer a single IEEE operation:
no contraction into fused multiply-add, no fast-math reassociation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "q4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra"]


def build(src=SRC, out=LIB, extra_flags=()):
    """Compile `src` into the shared library `out`; returns `out`."""
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


# AddressSanitizer + UndefinedBehaviorSanitizer build, with the ROCm clang so
# that it shares one sanitizer runtime with the HIP library's host code.
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_FLAGS = ["-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-fopenmp", "-Wall", "-Wextra", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def build_sanitized(out, src=SRC):
    """Compile `src` into `out` with ASan and UBSan (CPU checking of the oracle)."""
    tmp = out + ".tmp"
    subprocess.run([CLANG, *SAN_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
