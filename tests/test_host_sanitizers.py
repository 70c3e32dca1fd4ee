"""The library's host layer under AddressSanitizer and UndefinedBehavior-
Sanitizer, on the CPU: a build with both sanitizers on the host code (the
device code is never run) takes the place of libmoe.so in a child process
that runs the CPU tests which call into the library: every argument check
and error path of the C ABI (test_abi.py), the binding's validation
(test_api_validation.py) and the workspace sizes for many shapes
(test_resource_model.py).  Any invalid read or write, signed overflow,
misaligned access or shift out of range aborts the child."""
import os
import subprocess
import sys

import pytest

from mixture_experts_layer_exclusive_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKED = ["tests/test_abi.py", "tests/test_api_validation.py", "tests/test_resource_model.py"]


@pytest.fixture(scope="module")
def sanitized_lib(tmp_path_factory):
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not B.asan_runtime():
        pytest.skip("clang AddressSanitizer runtime not found")
    return B.build_host_sanitized(str(tmp_path_factory.mktemp("sanitized")))


def test_host_layer_is_clean_under_asan_and_ubsan(sanitized_lib):
    env = dict(os.environ)
    env.update(MOE_LIBRARY=sanitized_lib, LD_PRELOAD=B.asan_runtime(),
               # the interpreter's own allocations live until exit
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *CHECKED],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "passed" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]


def test_sanitized_library_is_the_one_loaded(sanitized_lib):
    # the child really loads the sanitized build (and ASan is initialised)
    env = dict(os.environ)
    env.update(MOE_LIBRARY=sanitized_lib, LD_PRELOAD=B.asan_runtime(), ASAN_OPTIONS="detect_leaks=0")
    code = ("import ctypes; from mixture_experts_layer_exclusive_amd import _lib as L; L.load(); "
            "import os; maps = open('/proc/self/maps').read(); "
            "print(L.LIB_PATH in maps, 'libclang_rt.asan' in maps, "
            "hasattr(ctypes.CDLL(None), '__asan_init'))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert r.stdout.split() == ["True", "True", "True"], r.stdout
