"""CPU safety net: the oracle's pin tests run against a gcc
AddressSanitizer + UndefinedBehaviorSanitizer build of the oracle, and the
host-side ABI tests run against a build of the HIP library whose host code
carries the same sanitizers.  Each suite runs in a child process with the
matching runtime preloaded; any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

import sanitize_build

HERE = os.path.dirname(os.path.abspath(__file__))
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer")


def _run_suite(test_file, env_extra, tmp_path):
    env = dict(os.environ)
    env.update(env_extra)
    # reports go to files: a child that dies on one cannot lose it in a pipe
    log = str(tmp_path / "san")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:log_path=" + log
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:log_path=" + log
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join(HERE, test_file)],
                         cwd=os.path.dirname(HERE), env=env, capture_output=True, text=True,
                         timeout=600)
    text = res.stdout + res.stderr
    reports = "".join(open(os.path.join(tmp_path, f)).read() for f in sorted(os.listdir(tmp_path))
                      if f.startswith("san"))
    assert not reports, reports[:4000]
    for r in REPORTS:
        assert r not in text, text[-4000:]
    assert res.returncode == 0, text[-4000:]
    return text


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = sanitize_build.oracle_lib()
    text = _run_suite("test_oracle.py", {"PA_ORACLE_LIB": lib,
                                         "LD_PRELOAD": sanitize_build.runtime("gcc")}, tmp_path)
    assert " passed" in text


def test_host_abi_under_asan_ubsan(tmp_path):
    lib = sanitize_build.hip_lib()
    text = _run_suite("test_abi_host.py", {"PA_LIBRARY": lib,
                                           "LD_PRELOAD": sanitize_build.runtime("clang")}, tmp_path)
    assert " passed" in text
