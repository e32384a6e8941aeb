"""Builds libkvarn.so (the HIP C-ABI library) in-tree for gfx950 with hipcc."""

import os
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
    build_c_client()
    return LIB


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


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
