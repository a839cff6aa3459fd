"""The host side of the C-ABI library under AddressSanitizer, on the CPU.

libqsa.so is rebuilt with its host code instrumented (-Xarch_host
-fsanitize=address; device code as usual) and the whole ABI test module runs
against that build in a child process with the ASan runtime preloaded: every
argument check, status path and host table construction it reaches runs
instrumented, and any heap or stack error aborts the child."""
import os
import subprocess
import sys

from block_sparse_long_qsa_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _env(lib):
    env = dict(os.environ)
    env.update(LD_PRELOAD=_build.ASAN_RUNTIME, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               QSA_LIB_PATH=lib, HIP_VISIBLE_DEVICES="")
    return env


def test_abi_tests_pass_under_host_asan():
    lib = _build.build_asan()
    env = _env(lib)
    # the runtime is live in the child and the binding loads the instrumented build
    probe = ("import ctypes, block_sparse_long_qsa_amd as Q; Q.lib(); "
             "assert Q.LIB_PATH == %r; assert hasattr(ctypes.CDLL(None), '__asan_report_load8')" % lib)
    r = subprocess.run([sys.executable, "-c", probe], env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr
