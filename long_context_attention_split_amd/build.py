"""Compile libtad.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m long_context_attention_split_amd.build

Objects go to ``_build/`` next to this file; the library to ``libtad.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtad.so")
# A plain HBM read stream that bench.py measures beside the split kernel; a
# measurement aid kept out of the decode library.
PROBE_LIB = os.path.join(HERE, "libtad_probe.so")

SOURCES = ["tad_api.cpp", "split_valu.hip", "split_mfma.hip", "split_heads.hip", "combine.hip"]
PROBE_SOURCES = ["stream_probe.hip"]

ARCH = "gfx950"
CFLAGS = [
    "-x", "hip", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    return os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + CFLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(ln for ln in r.stdout.splitlines() if "packed-fp32-ops" not in ln
                    and "not a recognized feature for this target" not in ln)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, out))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(PROBE_SOURCES))) as ex:
        objs = list(ex.map(_compile, srcs))
        probe_objs = list(ex.map(_compile, PROBE_SOURCES))
    ptmp = PROBE_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", ptmp] + probe_objs)
    os.replace(ptmp, PROBE_LIB)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    subprocess.check_call(cmd)
    # A kernel template the host pass could not instantiate leaves its launch stub
    # undefined without any diagnostic; such a library would only fail when loaded.
    nm = shutil.which("nm") or "/usr/bin/nm"
    undef = subprocess.run([nm, "-u", tmp], stdout=subprocess.PIPE, text=True, check=True).stdout
    stubs = [ln.split()[-1] for ln in undef.splitlines() if "__device_stub__" in ln]
    if stubs:
        os.remove(tmp)
        raise RuntimeError("kernel launch stubs left undefined by the host pass:\n  " + "\n  ".join(stubs))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, "and", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
