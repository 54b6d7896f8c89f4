"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code
that parses untrusted input: the bundle builder and image loader
(decode_gemv_amd/csrc/bundle.cpp, compiled with g++ on its own -- it holds no
GPU code) and the oracle (oracle/oracle.c, gcc).  Each is linked with a
driver under tests/sanitize/ that feeds it corrupted images or streams; the
sanitizers abort on any memory error or undefined behaviour.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:] + r.stderr[-4000:]
    return r


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_bundle_loader_under_sanitizers(tmp_path):
    exe = str(tmp_path / "bundle_fuzz")
    _run(["g++", "-std=c++17", *SAN, "-I" + os.path.join(ROOT, "include"),
          "-I" + os.path.join(ROOT, "decode_gemv_amd", "csrc"),
          os.path.join(ROOT, "decode_gemv_amd", "csrc", "bundle.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "bundle_fuzz.cpp"), "-o", exe, "-lpthread"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe, "1500"], env=env, timeout=600)
    assert "0 failed checks" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_fuzz")
    _run(["gcc", "-std=c11", *SAN, os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_fuzz.c"), "-o", exe, "-lm"])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = _run([exe, "200"], env=env, timeout=600)
    assert "0 failed checks" in r.stdout
