"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
the library is rebuilt with both sanitizers on its host pass (device code
unchanged) and tests/test_abi_cpu.py runs against it in a child process with
clang's ASan runtime preloaded.  Any report fails the test (halt_on_error,
reports written to files that must not exist afterwards).  No GPU is used."""

from __future__ import annotations

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


@pytest.mark.skipif(_asan_runtime() is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc or clang's ASan runtime not available")
def test_abi_validation_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from mla_latent_kv_06_amd import build
    lib = build.build_sanitized()
    logs = str(tmp_path / "san")
    env = dict(os.environ,
               LD_PRELOAD=_asan_runtime(),
               MLA_LIBRARY=lib,
               ASAN_OPTIONS=f"detect_leaks=0:alloc_dealloc_mismatch=0:new_delete_type_mismatch=0:"
                            f"halt_on_error=1:log_path={logs}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={logs}")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    reports = "".join(open(f).read() for f in glob.glob(logs + "*"))
    assert r.returncode == 0 and not reports, (r.stdout[-2000:], r.stderr[-2000:], reports[:4000])
    assert " passed" in r.stdout
