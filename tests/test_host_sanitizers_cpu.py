"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer: a
checking build (host code instrumented, device code unoptimised and never run) takes the
CPU tests of the C ABI (tests/test_abi_cpu.py: argument checks, status codes, workspace
and scratch queries, options) in a child process that preloads the sanitizer runtime.
Any report (an out-of-bounds or use-after-free access, an invalid enum or shift, a
signed overflow) ends the child with a non-zero status and a log file."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from accept_step_amd import build as libbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def asan_runtime(hipcc):
    r = subprocess.run([hipcc, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_abi_checks_are_clean_under_host_sanitizers(tmp_path):
    cmd = libbuild.hipcc_command(str(tmp_path / "libspecverify_san.so"), host_sanitizers=True)
    if shutil.which(cmd[0]) is None and not os.path.exists(cmd[0]):
        pytest.skip("hipcc is not installed")
    rt = asan_runtime(cmd[0])
    if rt is None:
        pytest.skip("the compiler's AddressSanitizer runtime is not installed")
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    logs = str(tmp_path / "san")
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    child = ("import sys\n"
             "import accept_step_amd as sv\n"
             f"sv.library_path = lambda: {str(tmp_path / 'libspecverify_san.so')!r}\n"
             "import pytest\n"
             "sys.exit(pytest.main(['tests/test_abi_cpu.py', '-q', '-p', 'no:cacheprovider']))\n")
    r = subprocess.run([sys.executable, "-c", child], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    assert r.returncode == 0 and not reports, (r.stdout[-3000:] + r.stderr[-2000:] + reports[:4000])
