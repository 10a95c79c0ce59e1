"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs
every pin without a report (no GPU).  A sanitizer finding (an out-of-bounds
access, a signed overflow, a misaligned load) aborts the child process."""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
       "-fno-omit-frame-pointer", "-g"]

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
from oracle import Oracle
from oracle_pins import ALL_PINS
orc = Oracle(lib_path={lib!r}, nthreads=2)
for pin in ALL_PINS:
    pin(orc)
    print("pin ok", pin.__name__, flush=True)
print("ALL_PINS_OK", flush=True)
"""


def _asan_runtime():
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_oracle_pins_under_asan_ubsan():
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "libcoli_oracle_san.so")
        oracle.build(out=lib, extra_flags=SAN)
        env = dict(os.environ, LD_PRELOAD=rt,
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=600)
    tail = (r.stdout[-2000:] + r.stderr[-4000:])
    assert r.returncode == 0 and "ALL_PINS_OK" in r.stdout, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail


HOST_CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import bit_gemv_coli_amd as coli
coli.LIB_PATH = {lib!r}
import pytest
sys.exit(int(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                          {test!r}])))
"""


def test_abi_host_checks_under_asan_ubsan():
    """The library's host side (argument validation, workspace sizing, the
    declines of every entry point) built with AddressSanitizer and
    UndefinedBehaviorSanitizer -- device code unchanged -- passes the host
    tests without a report.  No kernel is launched (no GPU here)."""
    import glob
    import shutil
    hipcc = shutil.which("hipcc")
    rts = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if hipcc is None or not rts:
        pytest.skip("hipcc or clang's AddressSanitizer runtime is missing")
    from bit_gemv_coli_amd import build as hb
    srcs = [os.path.join(hb.CSRC, s) for s in hb.SOURCES]
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", f]
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "libcoli_san.so")
        flags = [f for f in hb.FLAGS if f != "-O3"] + ["-O1", "-g"]
        subprocess.run([hipcc, *flags, *host_san, *srcs, "-o", lib], check=True,
                       capture_output=True, timeout=900)
        env = dict(os.environ, LD_PRELOAD=rts[0],
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        code = HOST_CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib,
                                 test=os.path.join(ROOT, "tests", "test_abi_host.py"))
        r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                           timeout=600)
    tail = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, tail
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, tail
