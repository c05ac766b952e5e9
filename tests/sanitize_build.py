"""Sanitizer builds for the CPU-side safety net (test infrastructure).

* the oracle's C source, built with gcc under AddressSanitizer and
  UndefinedBehaviorSanitizer (libpa_oracle_asan.so);
* the HIP library with the same two sanitizers on its host code only (the
  device code is compiled as in the release build): libpa_asan.so.

Both land in tests/_build (ignored by git).  `runtime(kind)` names the
sanitizer runtime a process must preload to load one of them.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "_build")
ORACLE_SRC = os.path.join(ROOT, "oracle", "pa_oracle.c")
CSRC = os.path.join(ROOT, "paged_attention_kv_pa_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SAN = ["address", "undefined"]


def oracle_lib() -> str:
    os.makedirs(OUT, exist_ok=True)
    out = os.path.join(OUT, "libpa_oracle_asan.so")
    cmd = (["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
            "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
           + ["-fsanitize=" + s for s in SAN] + ["-o", out, ORACLE_SRC, "-lm"])
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def _host(flag):
    return ["-Xarch_host", flag]


def hip_lib() -> str:
    os.makedirs(OUT, exist_ok=True)
    out = os.path.join(OUT, "libpa_asan.so")
    host = []
    for s in SAN:
        host += _host("-fsanitize=" + s)
    host += _host("-fno-omit-frame-pointer") + _host("-g") + _host("-shared-libsan")
    cmd = ([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fvisibility=hidden", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
           + host + ["-o", out] + sorted(glob.glob(os.path.join(CSRC, "*.hip"))))
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def runtime(kind: str) -> str:
    """Path of the ASan runtime to preload: 'gcc' for the oracle build, 'clang'
    for the HIP build."""
    if kind == "gcc":
        return subprocess.run(["gcc", "-print-file-name=libasan.so"], check=True,
                              capture_output=True, text=True).stdout.strip()
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not libs:
        raise FileNotFoundError("clang ASan runtime not found under /opt/rocm/llvm")
    return sorted(libs)[-1]
