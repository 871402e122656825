"""Compiles tests/c/abi_client.c (plain C, gcc) against include/normhip.h and
links it to the in-tree libnormhip.so and the HIP runtime.

    python tests/c/build_client.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_client.c")
EXE = os.path.join(HERE, "abi_client")
PKG = os.path.join(ROOT, "bwd_bn_stats_amd")
HEADER = os.path.join(ROOT, "include", "normhip.h")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(force: bool = False) -> str:
    deps = [SRC, HEADER, os.path.join(PKG, "libnormhip.so")]
    if not force and os.path.exists(EXE) and all(
            os.path.getmtime(EXE) >= os.path.getmtime(d) for d in deps if os.path.exists(d)):
        return EXE
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{ROOT}/include", f"-I{ROCM}/include", SRC, "-o", EXE + ".tmp",
           f"-L{PKG}", "-lnormhip", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{PKG}", "-Wl,-rpath,$ORIGIN/../../bwd_bn_stats_amd", f"-Wl,-rpath,{ROCM}/lib"]
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(force=True))
    sys.exit(0)
