"""Build libtropical.so: gfx950 code object + host runtime.

1. hipcc --genco compiles csrc/kernels/kernels.hip for gfx950 only.  Packed
   FP32 instructions are disabled (-packed-fp32-ops) and nothing enables
   fast math, FTZ or FMA contraction: every tropical term is one IEEE op.
2. The code object is embedded into the library with an assembler .incbin.
3. The host runtime (C++17, HIP runtime API only, no kernels) is compiled
   with g++ and linked against libamdhip64; its one source with device data
   (the allocation-free call's scratch array) is compiled by hipcc.

Output: tropical_semiring_tensor_amd/lib/libtropical.so (in-tree).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libtropical.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

ARCH = "gfx950"
DEVICE_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-fno-fast-math", "-ffp-contract=off", "-Wall"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter",
              "-D__HIP_PLATFORM_AMD__", "-I" + os.path.join(ROCM, "include")]
RUNTIME_SRCS = ["status.cpp", "module.cpp", "validate.cpp", "gemm.cpp", "gather.cpp", "contract.cpp",
                "backward.cpp", "tree.cpp"]
# host runtime sources with device data (compiled by hipcc, gfx950 only)
RUNTIME_HIP_SRCS = ["noalloc.hip"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("build step failed:\n  " + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res


def build_code_object(out=None):
    out = out or os.path.join(BUILD, "tropical_kernels.co")
    src = os.path.join(HERE, "kernels", "kernels.hip")
    _run([HIPCC, *DEVICE_FLAGS, "--genco", "--no-gpu-bundle-output", src, "-o", out])
    return out


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    co = os.path.join(BUILD, "tropical_kernels.co")
    blob = os.path.join(BUILD, "co_blob.S")

    def compile_host(name):
        obj = os.path.join(BUILD, name.replace(".cpp", ".o"))
        _run(["g++", *HOST_FLAGS, "-c", os.path.join(HERE, "runtime", name), "-o", obj])
        return obj

    def compile_hip_host(name):
        obj = os.path.join(BUILD, name.replace(".hip", ".o"))
        _run([HIPCC, "--offload-arch=" + ARCH, "-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-c", os.path.join(HERE, "runtime", name), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(RUNTIME_SRCS) + 2)) as ex:
        fut_co = ex.submit(build_code_object, co)
        fut_hip = [ex.submit(compile_hip_host, n) for n in RUNTIME_HIP_SRCS]
        objs = list(ex.map(compile_host, RUNTIME_SRCS))
        objs += [f.result() for f in fut_hip]
        fut_co.result()

    with open(blob, "w") as f:
        f.write(
            "    .section .rodata\n"
            "    .balign 4096\n"
            "    .globl trop_code_object\n"
            "    .type trop_code_object, @object\n"
            "trop_code_object:\n"
            f"    .incbin \"{co}\"\n"
            "    .globl trop_code_object_end\n"
            "trop_code_object_end:\n"
            "    .byte 0\n"
            "    .section .note.GNU-stack,\"\",@progbits\n")
    blob_obj = os.path.join(BUILD, "co_blob.o")
    _run(["gcc", "-c", blob, "-o", blob_obj])
    tmp = LIB + ".tmp"
    _run(["g++", "-shared", "-o", tmp, *objs, blob_obj, "-L" + os.path.join(ROCM, "lib"),
          "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-Wl,--no-undefined"])
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
