"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the sanitizer build (build.py --sanitize) runs the whole host ABI
suite -- packers and unpackers on exactly sized buffers, layout stamps, and the
argument checks of every entry point -- with no report; and a caller that
understates its buffer is caught, which shows the instrumentation is live."""
import os
import subprocess
import sys

import pytest

from moe_expert_gemv_amd import build

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def san_env():
    lib = build.build(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=build.sanitizer_runtime(), QG_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    yield env
    os.remove(lib)  # rebuilt by every run; not kept in the tree


def test_host_abi_suite_is_clean_under_sanitizers(san_env):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_host.py"],
                       env=san_env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in r.stdout


def test_sanitizer_catches_an_understated_buffer(san_env):
    """Negative control: the packer trusts dst_bytes, so a caller that claims
    more bytes than it allocated makes it write past the end -- ASan must
    report it (the library itself cannot see the real allocation)."""
    code = (
        "import ctypes, numpy as np, moe_expert_gemv_amd as qg\n"
        "L = qg.lib()\n"
        "codes = np.zeros((4, 64), np.uint8); scales = np.zeros((4, 4), np.uint8)\n"
        "need = qg.qg_packed_bytes(qg.QG_NVFP4, 4, 64)\n"
        "dst = np.zeros(need - 64, np.uint8)\n"
        "L.qg_pack_nvfp4(codes.ctypes.data, scales.ctypes.data, 4, 64, dst.ctypes.data, need)\n"
        "print('no report')\n")
    r = subprocess.run([sys.executable, "-c", code], env=san_env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stdout, r.stderr[-2000:])
    assert "heap-buffer-overflow" in r.stderr
