"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The oracle (oracle/qvref.c) is rebuilt with -fsanitize=address,undefined and its pin suite
  (tests/test_oracle.py) runs against that build.
* The ABI layer's host checks (qv_abi.cpp) are built with g++ under the same sanitizers, against
  a host-only stand-in of the HIP header and stub kernel launchers (tests/sanitize/), and the
  argument-error suite (tests/test_abi.py) runs against that library.
Any sanitizer report fails the run (halt_on_error, no recovery)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _runtime():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not path or not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    return path


def _env(log_dir, **extra):
    """Sanitizer reports go to files under log_dir (pytest's own capture of stderr would lose a
    report written just before the sanitizer ends the process)."""
    env = dict(os.environ, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log_dir}/asan",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log_dir}/ubsan")
    env.update(extra)
    return env


def _pytest(test_file, env, log_dir):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", test_file],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(os.path.join(log_dir, f)).read() for f in sorted(os.listdir(log_dir)))
    out = r.stdout + r.stderr
    assert not reports, reports[-3000:]
    assert r.returncode == 0, out[-3000:]
    return out


def test_oracle_under_sanitizers(tmp_path):
    from oracle.build import build_oracle

    _runtime()
    so = build_oracle(force=True, extra_flags=SAN, out=str(tmp_path / "libqvref_san.so"))
    logs = tmp_path / "logs"
    logs.mkdir()
    out = _pytest(os.path.join("tests", "test_oracle.py"), _env(logs, QVREF_LIB=so), logs)
    assert " passed" in out


def test_abi_checks_under_sanitizers(tmp_path):
    _runtime()
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(ROOT, "bit_ptq_reconstruction_amd", "csrc")
    so = str(tmp_path / "libqv_abi_stub.so")
    cmd = ["g++", "-std=c++17", "-O1", "-shared", "-fPIC", "-Wall", *SAN,
           "-I", os.path.join(ROOT, "tests", "sanitize"),  # the host-only HIP header comes first
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "qv_abi.cpp"), os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"), "-o", so]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    logs = tmp_path / "logs"
    logs.mkdir()
    out = _pytest(os.path.join("tests", "test_abi.py"), _env(logs, QV_ABI_TEST_LIB=so), logs)
    assert " passed" in out and "skipped" not in out
