"""Host-side validation of the C ABI, and the C oracle, under AddressSanitizer and
UndefinedBehaviorSanitizer.

Both host layers are rebuilt with the sanitizers on host code only: tad_api.cpp
through hipcc with every sanitizer flag behind -Xarch_host (its kernels come from
the ordinary objects of the in-tree build), and decode_f64.c through clang. A
child process then runs the host ABI tests and the oracle's pins against those
builds, with the sanitizer runtime preloaded into the interpreter. An invalid
read or write, or any undefined behaviour (signed overflow, a misaligned or null
access, an out-of-range shift), stops the child and fails this test.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_attention_split_amd")
CSRC = os.path.join(PKG, "csrc")
OBJS = ["split_valu.o", "split_mfma.o", "split_heads.o", "combine.o"]

# The child runs the tests, then checks that the sanitized builds are the ones mapped.
CHILD = r"""
import os, sys, pytest
rc = pytest.main(sys.argv[1:])
maps = open("/proc/self/maps").read()
for env in ("TAD_LIB_PATH", "ORACLE_LIB_PATH"):
    if os.environ[env] not in maps:
        print("not loaded:", os.environ[env]); rc = rc or 3
sys.exit(int(rc))
"""


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stdout[-4000:])
    return r.stdout


def _undefined(lib):
    nm = shutil.which("nm") or "/usr/bin/nm"
    return _run([nm, "-D", "-u", lib])


def test_host_layers_under_asan_and_ubsan(lib, tmp_path):
    rt = _runtime()
    if rt is None:
        pytest.skip("no clang AddressSanitizer runtime under /opt/rocm/llvm")
    from long_context_attention_split_amd import build as b
    objs = [os.path.join(b.BUILD, o) for o in OBJS]
    missing = [o for o in objs if not os.path.exists(o)]
    assert not missing, "run the in-tree build first: %s" % missing

    host_san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                 "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", flag]
    api_o = str(tmp_path / "tad_api_san.o")
    _run([b.hipcc()] + b.CFLAGS + ["-g"] + host_san + ["-c", os.path.join(CSRC, "tad_api.cpp"), "-o", api_o])
    tad_so = str(tmp_path / "libtad_san.so")
    rtdir = os.path.dirname(rt)
    _run(["g++", "-shared", "-fPIC", "-o", tad_so, api_o] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", rt, "-Wl,-rpath," + rtdir,
          "-Wl,--no-undefined"])

    oracle_so = str(tmp_path / "liboracle_san.so")
    clang = "/opt/rocm/llvm/bin/clang"
    _run([clang, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-shared-libsan",
          os.path.join(ROOT, "oracle", "decode_f64.c"), "-o", oracle_so, "-lm", "-Wl,-rpath," + rtdir])

    # Both builds really are instrumented.
    for so in (tad_so, oracle_so):
        und = _undefined(so)
        assert "__asan_report_" in und and "__ubsan_handle_" in und, so

    env = dict(os.environ)
    env.update(TAD_LIB_PATH=tad_so, ORACLE_LIB_PATH=oracle_so, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=86",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=87")
    out = _run([sys.executable, "-c", CHILD, "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                os.path.join(ROOT, "tests", "test_abi_host.py"),
                os.path.join(ROOT, "tests", "test_oracle_pins.py")], env=env, cwd=str(tmp_path))
    assert " passed" in out and "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-2000:]
