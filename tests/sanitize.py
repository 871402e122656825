"""Host-sanitizer run of the CPU test suite.

    python tests/sanitize.py [extra pytest arguments]

Builds, under _build/san/, a copy of the oracle (oracle.c) and of the
library (every source; only the host side instrumented: AddressSanitizer and
UndefinedBehaviorSanitizer, the GPU code compiled as usual), then runs
`pytest -m "not gpu"` with both copies in place of the in-tree ones
(ORACLE_LIBRARY, NORMHIP_LIBRARY, and LD_LIBRARY_PATH for the plain-C ABI
client) and the sanitizer runtime preloaded into the interpreter.  Any
sanitizer report ends the run with a non-zero status.  Runs on the CPU only;
the suite's GPU tests stay deselected.

Both copies use clang's sanitizer runtime (one runtime per process), so the
oracle is compiled here by ROCm's clang with its OpenMP runtime instead of
gcc.  Leak checking is off: the interpreter and the HIP runtime keep their
allocations until exit.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(ROOT, "_build", "san")
LLVM = "/opt/rocm/llvm"

# host-only instrumentation on the hipcc lines; plain options for clang's C build
HIP_HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split() + \
    "-Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=undefined".split()
HIP_LINK_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split() + ["-shared-libasan"]
C_SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined",
         "-shared-libasan", f"-L{LLVM}/lib", f"-Wl,-rpath,{LLVM}/lib"]


def asan_runtime() -> str:
    found = sorted(glob.glob(f"{LLVM}/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise SystemExit("clang's AddressSanitizer runtime was not found under " + LLVM)
    return found[-1]


def build() -> tuple[str, str]:
    sys.path.insert(0, ROOT)
    os.makedirs(OUT, exist_ok=True)
    import oracle
    from bwd_bn_stats_amd import build as hipbuild
    olib = oracle.build(force=True, cc=f"{LLVM}/bin/clang", extra_flags=C_SAN,
                        out=os.path.join(OUT, "liboracle.so"))
    nlib = hipbuild.build(verbose=True, extra_flags=HIP_HOST_SAN, link_flags=HIP_LINK_SAN,
                          lib=os.path.join(OUT, "libnormhip.so"), build_dir=os.path.join(OUT, "obj"))
    return olib, nlib


def main(argv) -> int:
    olib, nlib = build()
    env = dict(os.environ)
    env.update({
        "ORACLE_LIBRARY": olib,
        "NORMHIP_LIBRARY": nlib,
        "LD_LIBRARY_PATH": OUT + (":" + env["LD_LIBRARY_PATH"] if env.get("LD_LIBRARY_PATH") else ""),
        "LD_PRELOAD": asan_runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    # the interpreter and the C client must map the instrumented copies
    probe = ("import sys; sys.path.insert(0, %r); import oracle; oracle._load(); "
             "from bwd_bn_stats_amd import normhip; "
             "maps = open('/proc/self/maps').read(); "
             "assert %r in maps and %r in maps and 'libclang_rt.asan' in maps, 'not the sanitized libraries'; "
             "print('preflight: sanitized oracle and library loaded')" % (ROOT, olib, nlib))
    if subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT).returncode != 0:
        return 1
    sys.path.insert(0, os.path.join(HERE, "c"))
    import build_client
    ldd = subprocess.run(["ldd", build_client.build(force=True)], env=env, capture_output=True, text=True).stdout
    if nlib not in ldd:
        print("the C client does not resolve the sanitized library:\n" + ldd)
        return 1
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-x", "-q", "-m", "not gpu",
           "-p", "no:cacheprovider", *argv]
    print("sanitized run:", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
