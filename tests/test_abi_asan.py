"""The host-side ABI checks again, against a copy of the library whose host
code is built with AddressSanitizer (device code as usual).

Argument validation (sequence ranges, overlap tests, workspace sizes) is host
code that runs on every call; under ASan any out-of-bounds or use-after-free
access in it aborts the run. The ASan runtime is preloaded into a child
Python that runs tests/test_abi_host.py with ZEBRA_LIBRARY pointing at the
sanitized build. Nothing here launches a kernel.
"""

import os
import subprocess
import sys

import pytest

from linear_hybrid_attention_zebra_amd import build as zbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    try:
        path = zbuild.asan_runtime()
    except Exception:  # pragma: no cover - no toolchain
        return None
    return path if path and os.path.exists(path) else None


@pytest.mark.skipif(_runtime() is None, reason="no host AddressSanitizer runtime")
def test_host_abi_checks_under_asan():
    lib = zbuild.build_asan()
    env = dict(os.environ, ZEBRA_LIBRARY=lib, LD_PRELOAD=_runtime(),
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:halt_on_error=1")
    probe = subprocess.run(
        [sys.executable, "-c",
         "import linear_hybrid_attention_zebra_amd as zb; zb.library(); "
         "m = open('/proc/self/maps').read(); "
         "print(int('libclang_rt.asan' in m), int('libzebra_asan.so' in m))"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.stdout.split()[-2:] == ["1", "1"], probe.stdout + probe.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join("tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout[-4000:] + res.stderr[-4000:]
    assert "AddressSanitizer" not in res.stderr, out
    assert res.returncode == 0, out
    assert " passed" in res.stdout, out
