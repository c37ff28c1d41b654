"""Build libspmm_csr_spmv.so (hipcc, gfx950) in the package directory.

Usage: python -m spmm_csr_spmv_amd.build   (or __graft_entry__.build()).
Every call recompiles; objects are placed in _build/ beside the package.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libspmm_csr_spmv.so")
# measurement probe loaded only by bench.py (not part of the library's ABI)
PROBE_LIB = os.path.join(HERE, "libspx_probe.so")
PROBE_SOURCES = ["probe.hip"]

SOURCES = ["api.cpp", "plan_host.cpp", "tune.cpp", "convert.hip", "spmv.hip", "pstream.hip", "spmm.hip", "bsr.hip", "bsr_convert.hip", "wcsr.hip", "xwin.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I" + INCLUDE, "-I" + CSRC,
          "--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + lang + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-pthread", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(verbose=False):
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
