"""The host code — argument validation of every entry point and the native
block manager — under AddressSanitizer and UndefinedBehaviorSanitizer: the
library is rebuilt with both on its host pass (device code unchanged) and the
GPU-free ABI and block-manager tests run against it in a child process, any
sanitizer report failing them.  CPU only: on a machine with a GPU the child
would start the HIP runtime under the sanitizer's preload, so it is skipped
there."""

import glob
import os
import shutil
import subprocess
import sys

import pytest

from conftest import ROOT, gpu_available

CLANG = "/opt/rocm/llvm/bin/clang"


def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    if gpu_available():
        pytest.skip("runs on machines without a GPU")
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")) or not os.path.exists(CLANG):
        pytest.skip("hipcc / clang not found")
    runtime = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                             capture_output=True, text=True).stdout.strip()
    if not os.path.isfile(runtime):
        pytest.skip("AddressSanitizer runtime not found")
    sys.path.insert(0, ROOT)
    from paged_kv_cache_248_amd.build import build
    lib = build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=runtime, PA_LIBRARY=lib,
               ASAN_OPTIONS=f"detect_leaks=0:log_path={tmp_path}/report",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p",
                        "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_block_manager.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = [open(f).read() for f in glob.glob(f"{tmp_path}/report*")]
    assert not reports, "sanitizer report:\n" + "\n".join(x[:4000] for x in reports)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
