"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two programs are built with the host compilers and the sanitizers on, with
no recovery (the first report aborts the run):

* tests/sanitize/host_check.cpp against the library's host unit
  (quant_verify_gemv_amd/csrc/kq_api.cpp) and host-only stand-ins for its
  kernel launchers (tests/sanitize/kernel_stubs.cpp, which also check each
  launch description against the invariants the kernels rely on): every
  C-ABI entry point through its argument checks, the size functions over
  edge shapes, the chain encode / status path, and the host decision with
  the MT19937 stream on random inputs.
* tests/sanitize/oracle_check.c against the oracle (oracle/kq_oracle.c,
  with OpenMP): every oracle function on random and edge inputs.

Each program prints one summary line and exits 0 only when all of its
expectations hold and no sanitizer reported anything."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")


def _build(cmd, tmp_path):
    r = subprocess.run(cmd, cwd=tmp_path, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    if r.returncode != 0 and ("cannot find -lasan" in r.stdout or "cannot find -lubsan" in r.stdout):
        pytest.skip("the host compiler has no sanitizer runtime")
    assert r.returncode == 0, r.stdout[-4000:]


def _run(exe, tmp_path):
    r = subprocess.run([exe], cwd=tmp_path, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600, env=ENV)
    assert r.returncode == 0, r.stdout[-6000:]
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error" not in r.stdout, r.stdout[-6000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no g++")
def test_host_library_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_check")
    _build(["g++", "-std=c++17", *FLAGS, "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(ROOT, "quant_verify_gemv_amd", "csrc"), "-I", SAN,
            os.path.join(ROOT, "quant_verify_gemv_amd", "csrc", "kq_api.cpp"),
            os.path.join(SAN, "kernel_stubs.cpp"), os.path.join(SAN, "host_check.cpp"), "-o", exe], tmp_path)
    out = _run(exe, tmp_path)
    assert ", 0 failed;" in out, out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _build(["gcc", "-std=c11", "-fopenmp", *FLAGS, os.path.join(ROOT, "oracle", "kq_oracle.c"),
            os.path.join(SAN, "oracle_check.c"), "-lm", "-o", exe], tmp_path)
    out = _run(exe, tmp_path)
    assert ", 0 failed" in out, out
