"""Builds libkvarn.so (the HIP C-ABI library) in-tree for gfx950 with hipcc."""

import os
import shlex
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvarn.so")
SOURCES = ["kvarn_api.hip", "kvarn_quantize.hip", "kvarn_decode.hip"]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libkvarn.so; returns the library path."""
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Wno-unused-result",
           # keep the compiler from emitting packed-fp32 instructions
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(HERE, "..", "include"),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", LIB + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkvarn.so")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(LIB + ".tmp", LIB)
    build_probe()
    build_c_client()
    build_asan_client()
    return LIB


PROBE_LIB = os.path.join(HERE, "libkvarn_probe.so")


def build_probe() -> str:
    """The read-only HBM streaming probe (benchmark context only; not part of the C ABI)."""
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, "kvarn_probe.hip"), "-o", PROBE_LIB + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libkvarn_probe.so")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


C_CLIENT_SRC = os.path.join(HERE, "..", "tests", "c", "kvarn_c_client.c")
C_CLIENT = os.path.join(HERE, "..", "tests", "c", "kvarn_c_client")          # host checks only
C_CLIENT_GPU = os.path.join(HERE, "..", "tests", "c", "kvarn_c_client_gpu")  # + HIP runtime


def build_c_client() -> None:
    """The plain C99 test client of the C ABI (gcc), once without and once with the HIP
    runtime's C API; both link libkvarn.so from this directory."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    inc = os.path.join(HERE, "..", "include")
    common = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-I", inc, C_CLIENT_SRC,
              "-L", HERE, "-lkvarn", "-Wl,-rpath," + HERE]
    for out, extra in ((C_CLIENT, ["-pedantic"]),
                       (C_CLIENT_GPU, ["-DKVARN_C_CLIENT_GPU", "-D__HIP_PLATFORM_AMD__", "-I",
                                       os.path.join(rocm, "include"), "-L",
                                       os.path.join(rocm, "lib"), "-lamdhip64",
                                       "-Wl,-rpath," + os.path.join(rocm, "lib")])):
        res = subprocess.run(common[:1] + extra[:1] + common[1:] + extra[1:] + ["-o", out],
                             capture_output=True, text=True)
        if res.returncode != 0:      # a test client: its tests skip without it
            sys.stderr.write(res.stdout + res.stderr)
            sys.stderr.write("warning: gcc failed building " + os.path.basename(out) + "\n")


C_CLIENT_ASAN = os.path.join(HERE, "..", "tests", "c", "kvarn_c_client_asan")
# AddressSanitizer for host code only: -Xarch_host before each sanitizer flag keeps it out of
# the gfx950 device code
ASAN_HOST_FLAGS = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer")
ASAN_DIR = os.path.join(HERE, "..", "_build", "asan")


def build_asan_client() -> str:
    """The C client's host checks linked with a copy of the library whose host code carries
    AddressSanitizer (clang's runtime; the device code is built as usual). Returns its path, or
    '' when the toolchain cannot build it (its test then skips)."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    os.makedirs(ASAN_DIR, exist_ok=True)
    inc = os.path.join(HERE, "..", "include")
    objs = []
    for src in SOURCES:
        obj = os.path.join(ASAN_DIR, src.replace(".hip", ".o"))
        cmd = [hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
               *ASAN_HOST_FLAGS, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", inc, "-c",
               os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr + "warning: ASan build skipped\n")
            return ""
        objs.append(obj)
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    cobj = os.path.join(ASAN_DIR, "kvarn_c_client.o")
    steps = [[clang, "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror", *ASAN_HOST_FLAGS,
              "-I", inc, "-c", C_CLIENT_SRC, "-o", cobj],
             [hipcc(), "--offload-arch=gfx950", *ASAN_HOST_FLAGS, *objs, cobj, "-o", C_CLIENT_ASAN]]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr + "warning: ASan build skipped\n")
            return ""
    return C_CLIENT_ASAN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
