"""Builds libpa.so (the HIP library behind include/pa.h) in-tree for gfx950, and
libpa_debug.so: the same library compiled with PA_DEBUG, whose kernels check
every block-table entry against the page pool (an entry outside it is reported
as PA_ERR_DEVICE_DATA instead of being read) and whose calls wait for their
stream to report it."""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libpa.so")
DEBUG_LIB = os.path.join(PKG, "libpa_debug.so")
ARCH = "gfx950"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _flags(debug: bool):
    f = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-I" + INCLUDE, "-I" + CSRC,
         # packed fp32 instructions stay off for every kernel of this library
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    return f + (["-DPA_DEBUG"] if debug else [])


def command(out_path: str, debug: bool = False):
    """One hipcc command that compiles and links every source (for reference)."""
    return [_hipcc()] + _flags(debug) + ["-shared", "-o", out_path] + sources()


def _filter(text):
    return "\n".join(l for l in text.splitlines()
                     if "packed-fp32-ops" not in l and "argument unused during compilation" not in l)


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return res.returncode, _filter(res.stdout)


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every HIP source (one process per source) and link the library
    (always rebuilds).  debug: build libpa_debug.so with PA_DEBUG."""
    out = DEBUG_LIB if debug else LIB
    tag = "d" if debug else "r"
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(objdir, "%s_%s_%d.o" % (os.path.basename(src)[:-4], tag, os.getpid()))
        objs.append(obj)
        cmds.append([_hipcc()] + _flags(debug) + ["-c", src, "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, text) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError("hipcc failed:\n" + text)
        if verbose and text.strip():
            print(text)
    tmp = out + ".tmp%d" % os.getpid()
    rc, text = _run([_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    for o in objs:
        os.remove(o)
    if rc != 0:
        raise RuntimeError("link failed:\n" + text)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
