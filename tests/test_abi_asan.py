"""The host-side ABI tests (argument checks, error paths, the binding's
marshalling) under AddressSanitizer: the library is rebuilt with ASan on its
host code (device code unchanged) and the tests run in a subprocess with the
ASan runtime preloaded.  Runs without a GPU."""
import glob
import os
import subprocess
import sys

import pytest

from weight_quantized_moe_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib):
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    srcs = build.sources() + glob.glob(os.path.join(ROOT, "include", "*.h")) + \
        glob.glob(os.path.join(build.CSRC, "*.h"))
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.mark.timeout(900)
def test_abi_under_address_sanitizer():
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if _stale(build.ASAN_LIB):
        build.build_asan()
    env = dict(os.environ, MOE_QUANT_LIB=build.ASAN_LIB, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py"),
                          os.path.join(ROOT, "tests", "test_binding_checks.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "AddressSanitizer" not in res.stderr, tail
