"""Builds libw4a16.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m w4a16_dequant_gemv_amd.build

Every translation unit is compiled with packed-fp32 instruction selection
disabled; the weight quantizer's, the KV codec's, the W8A8 and the GPTQ/AWQ units
additionally keep
each fp32 operation separate (no FMA contraction) and use correctly rounded
fp32 division, which their bit-exactness depends on.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libw4a16.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
EXACT_FP32 = ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math"]
PER_FILE = {
    "q4_quantize.hip": EXACT_FP32,
    "kv_codec.hip": EXACT_FP32,
    "w8a8.hip": EXACT_FP32,
    "producers.hip": EXACT_FP32,
}
SOURCES = ["q4_api.hip", "q4_quantize.hip", "q4_gemv.hip", "q4_gemm.hip", "kv_codec.hip", "w8a8.hip",
           "producers.hip"]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (argument checking,
# dispatch, launch code); the device code is compiled as usual.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


def _compile(src, build_dir=BUILD_DIR, extra=()):
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature; that
    # warning is expected and dropped here.
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose=True):
    """Compile every source and link libw4a16.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                   check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def build_host_sanitized(out, build_dir):
    """libw4a16 with ASan/UBSan on its host code, linked to `out` (objects in
    `build_dir`); load it with the clang ASan runtime preloaded."""
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, HOST_SANITIZE), SOURCES))
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", out, *objs], check=True)
    return out


if __name__ == "__main__":
    build()
