"""The host side of the library (argument validation, workspace sizing, dispatch
and the no-device error paths) under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the checking variant of libattn.so (host code instrumented, device code
untouched; rebuilt when a source is newer than it), then runs the C-ABI suite
(tests/test_abi.py) in a child process that loads it, with the shared ASan
runtime preloaded and every UBSan finding fatal. CPU only: without a device the
calls that pass validation end in their HIP error path, which is checked too.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from transformer_attention_02_amd import build as B  # noqa: E402


def _asan_runtime():
    clang = "/opt/rocm/llvm/bin/clang"
    if not os.path.exists(clang):
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _stale(lib):
    if not os.path.exists(lib):
        return True
    srcs = glob.glob(os.path.join(B.CSRC, "*")) + [os.path.join(ROOT, "include", "attn.h")]
    return max(os.path.getmtime(s) for s in srcs) > os.path.getmtime(lib)


@pytest.mark.timeout(900)
def test_abi_suite_is_clean_under_asan_and_ubsan():
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a preload is already in place; it is left alone")
    rt = _asan_runtime()
    if rt is None or shutil.which(B.hipcc()) is None:
        pytest.skip("no ASan runtime / hipcc")
    if _stale(B.SAN_LIB):
        B.build_library(sanitize=True)
    env = dict(os.environ, ATTN_LIB=B.SAN_LIB, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
