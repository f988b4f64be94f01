"""The host side of liboctopus.so under AddressSanitizer and
UndefinedBehaviorSanitizer.

The library's host code (descriptor and cache-view validation, bit-split
resolution, workspace sizing, the error paths of every entry point) is
built with -fsanitize=address,undefined (build.py --sanitize, host
compilation only) into liboctopus_san.so, and the ABI checks of
tests/test_abi.py and tests/test_binding_checks.py are run against it in a
child process with the sanitizer runtime preloaded.  Any report (an
out-of-bounds access, a load of an invalid enum value, a signed overflow,
...) aborts that process and fails this test.  No kernel is launched.
"""
import os
import subprocess
import sys

import pytest

from quantized_decode_attention_octo_amd import build as ob_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHECKS = ["tests/test_abi.py", "tests/test_binding_checks.py"]


def _stale():
    if not os.path.exists(ob_build.LIB_SAN):
        return True
    t = os.path.getmtime(ob_build.LIB_SAN)
    srcs = [os.path.join(ob_build.CSRC, f) for f in os.listdir(ob_build.CSRC)]
    srcs += [os.path.join(ob_build.INCLUDE, f) for f in os.listdir(ob_build.INCLUDE)]
    return any(os.path.getmtime(s) > t for s in srcs)


@pytest.fixture(scope="module")
def san_env():
    try:
        runtime = ob_build.sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    if _stale():
        ob_build.build(sanitize=True)
    env = dict(os.environ)
    env.update(OCTO_LIB=ob_build.LIB_SAN, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def test_sanitized_library_is_the_one_loaded(san_env):
    code = ("from quantized_decode_attention_octo_amd import binding as b; b.lib(); "
            "print(any('liboctopus_san.so' in l for l in open('/proc/self/maps')))")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=san_env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip().endswith("True")


def test_abi_checks_under_asan_and_ubsan(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + CHECKS,
                       cwd=ROOT, env=san_env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
