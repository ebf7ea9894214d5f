"""The host-side C ABI checks (tests/test_abi_cpu.py) again, against a build of libcsa2 whose
host layer (api.cpp: descriptor validation, workspace sizing, error reporting, the
no-allocation entry point's scratch lookup) is instrumented with AddressSanitizer and
UndefinedBehaviorSanitizer.  The kernels are the ordinary objects; no GPU is used.

The checks run in a child process with the ASan runtime preloaded (the interpreter itself is
not instrumented) and any sanitizer report fatal, so an out-of-bounds access or undefined
behaviour in the validation paths fails this test."""
import os
import subprocess
import sys

import pytest

from compressed_sparse_attention_gated_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def env():
    rt = B.sanitizer_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this toolchain")
    lib = B.build_sanitized()
    e = dict(os.environ)
    e.update(LD_PRELOAD=rt, LD_LIBRARY_PATH=os.path.dirname(rt) + ":" + e.get("LD_LIBRARY_PATH", ""),
             CSA2_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
             UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return e


def test_sanitized_library_is_the_one_loaded(env):
    code = ("import torch\nfrom compressed_sparse_attention_gated_amd import csa2\ncsa2.lib()\n"
            "print([l.split()[-1] for l in open('/proc/self/maps') if 'libcsa2' in l][0])")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.strip() == B.SANITIZE_LIB


def test_abi_checks_under_asan_and_ubsan(env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
