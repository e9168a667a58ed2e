"""Builds the in-tree shared libraries with hipcc for gfx950.

libhas.so    the product: C ABI of include/has.h (HIP kernels + host code)
libsynth.so  the seeded input generator (host + device fill), test/bench input
tests/_build/libhas_san.so
             the same sources with AddressSanitizer and UndefinedBehavior-
             Sanitizer on the host code (device code as usual), for the CPU
             tests of the argument validation
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "head_aware_sparse_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-shared", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

HAS_SOURCES = [os.path.join(PKG, "csrc", f) for f in ("api.cpp", "decode.hip", "label.hip")]
HAS_LIB = os.path.join(PKG, "libhas.so")
SYNTH_SOURCES = [os.path.join(ROOT, "synth", "csrc", "synth.hip")]
SYNTH_LIB = os.path.join(ROOT, "synth", "libsynth.so")


def _run(cmd):
    print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError(f"build failed: {cmd[-1]}")
    if out.strip():
        print(out)


def build_has():
    cmd = [HIPCC, *COMMON, "-I", os.path.join(ROOT, "include"), "-x", "hip", *HAS_SOURCES,
           "-o", HAS_LIB + ".tmp"]
    # api.cpp carries no device code, but compiling it as HIP keeps one toolchain.
    _run(cmd)
    os.replace(HAS_LIB + ".tmp", HAS_LIB)


def build_synth():
    _run([HIPCC, *COMMON, "-ffp-contract=off", *SYNTH_SOURCES, "-o", SYNTH_LIB + ".tmp"])
    os.replace(SYNTH_LIB + ".tmp", SYNTH_LIB)


SAN_LIB = os.path.join(ROOT, "tests", "_build", "libhas_san.so")
# sanitizers on the host pass only (-Xarch_host before each): the kernels are
# built as in the product, the validation and launch code is instrumented;
# undefined behaviour aborts instead of printing and continuing
SAN_FLAGS = ["-O1", "-g", "-fPIC", "-shared", "-std=c++17", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libsan",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def build_has_sanitized():
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    _run([HIPCC, *SAN_FLAGS, "-I", os.path.join(ROOT, "include"), "-x", "hip", *HAS_SOURCES, "-o", SAN_LIB + ".tmp"])
    os.replace(SAN_LIB + ".tmp", SAN_LIB)


def asan_runtime():
    """The clang AddressSanitizer runtime the sanitized library links to."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_all():
    build_synth()
    build_has()
    build_has_sanitized()


if __name__ == "__main__":
    build_all()
