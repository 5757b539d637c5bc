"""Host-only build of the library's pure C++ parts with AddressSanitizer and
UndefinedBehaviorSanitizer: the block manager (zp_bm_*), the hybrid scheduler
(zp_sched_*) and the error text. No GPU code is compiled (g++ only).

build() returns the path of _build/host_sanitize/libzipage_host.so; run(...)
runs pytest arguments in a child Python process with the sanitizer runtimes
preloaded and ZIPAGE_LIB pointing the binding at that build.

Usage: python -m kv_cache_compression_paged_amd.host_sanitize [pytest args]
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(ROOT, "_build", "host_sanitize")
LIB = os.path.join(OUT, "libzipage_host.so")
HOST_SOURCES = ["block_manager.cpp", "scheduler.cpp", "errors.cpp"]
FLAGS = ["-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]


def build() -> str:
    os.makedirs(OUT, exist_ok=True)
    cmd = (["g++"] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
           + [os.path.join(CSRC, s) for s in HOST_SOURCES] + ["-o", LIB])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"host sanitizer build failed:\n{res.stderr}")
    return LIB


def runtime_libs() -> list:
    out = []
    for name in ("libasan.so", "libubsan.so"):
        path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                              text=True, check=True).stdout.strip()
        out.append(path)
    return out


def run(pytest_args: list, timeout: float = 600) -> subprocess.CompletedProcess:
    lib = build()
    env = dict(os.environ)
    env["ZIPAGE_LIB"] = lib
    env["LD_PRELOAD"] = ":".join(runtime_libs())
    # the interpreter itself is not instrumented: leaks of its own are not ours
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider"]
                          + pytest_args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


if __name__ == "__main__":
    r = run(sys.argv[1:])
    sys.stdout.write(r.stdout[-4000:])
    sys.stderr.write(r.stderr[-4000:])
    sys.exit(r.returncode)
