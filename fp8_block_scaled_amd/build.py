"""Build libfp8bs.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc.

    python -m fp8_block_scaled_amd.build          # or fp8_block_scaled_amd.build.build()

Objects go to fp8_block_scaled_amd/_build/, the library to
fp8_block_scaled_amd/libfp8bs.so.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfp8bs.so")
# Measurement kernels of the bench (stream read, MFMA loop, shader clock): a library of
# their own, not part of the product ABI.
CEIL_LIB = os.path.join(PKG, "libfp8bs_ceilings.so")
SOURCES = ["api.hip", "quant.hip", "gemm_decode.hip", "gemm_mid.hip", "gemm_prefill.hip", "w4a16.hip", "splitk.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # No packed FP32 instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE float32 division and FP32 denormals: the quantizer is bit-exact only with both.
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=fast",
    "-Wall",
    "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, jobs=None):
    """Compile every HIP source for gfx950 and link libfp8bs.so.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        _run([HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        return obj

    with ThreadPoolExecutor(jobs or min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    tmp = CEIL_LIB + ".tmp"
    _run([HIPCC, *CFLAGS, "-shared", os.path.join(CSRC, "ceilings.hip"), "-o", tmp], verbose)
    os.replace(tmp, CEIL_LIB)
    return LIB


SAN_LIB = os.path.join(BUILD, "libfp8bs_hostsan.so")


def sanitizer_runtime():
    """The clang AddressSanitizer runtime (it carries UBSan too) that a process loading
    the host-sanitized library must preload."""
    rocm_llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "llvm")
    clang_dir = os.path.join(rocm_llvm, "lib", "clang")
    for ver in sorted(os.listdir(clang_dir), reverse=True) if os.path.isdir(clang_dir) else []:
        p = os.path.join(clang_dir, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    raise RuntimeError("clang AddressSanitizer runtime not found")


def build_sanitized_abi(verbose=False):
    """Build a second copy of the library whose host code in api.hip (argument
    validation, device check, schedule choice) is instrumented with AddressSanitizer
    and UndefinedBehaviorSanitizer; device code and the other sources are the normal
    objects.  tests/test_abi_sanitized.py runs the ABI validation tests against it on
    the CPU.  Needs build() first (it links build()'s objects)."""
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, "api_hostsan.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in CFLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([HIPCC, *flags, *san, "-c", os.path.join(CSRC, "api.hip"), "-o", obj], verbose)
    objs = [os.path.join(BUILD, src.replace(".hip", ".o")) for src in SOURCES if src != "api.hip"]
    tmp = SAN_LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, *objs, "-shared-libsan",
          "-fsanitize=address,undefined", "-o", tmp], verbose)
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


C_ABI_SRC = os.path.join(ROOT, "tests", "c_abi", "abi_roundtrip.c")
C_ABI_BIN = os.path.join(ROOT, "tests", "c_abi", "abi_roundtrip")


def build_c_abi_check(verbose=False):
    """Compile the plain-C caller of the ABI (host code only, gcc) against libfp8bs.so;
    a GPU test runs it.  Needs the library built first."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for the ABI check")
    _run([cc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{os.path.join(ROOT, 'include')}",
          f"-I{os.path.join(rocm, 'include')}", C_ABI_SRC, f"-L{PKG}", "-lfp8bs", f"-L{os.path.join(rocm, 'lib')}",
          "-lamdhip64", "-lm", "-Wl,-rpath,$ORIGIN/../../fp8_block_scaled_amd",
          f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", C_ABI_BIN], verbose)
    return C_ABI_BIN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_c_abi_check(verbose="-v" in sys.argv))
    print(build_sanitized_abi(verbose="-v" in sys.argv))
