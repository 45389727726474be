"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer:
a sanitized build of mxq_oracle.c runs every pin in a child process (the
sanitizer runtimes are preloaded there), which must finish cleanly."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
oracle._DEFAULT = oracle.Oracle({lib!r})
from pins import ALL_PINS
orc = oracle.default()
for p in ALL_PINS:
    p(orc)
print("pins ok", len(ALL_PINS))
"""


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the oracle")
def test_pins_under_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "liboracle_san.so")
        subprocess.run(oracle.build_command(out=lib, extra=("-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                                                            "-fno-omit-frame-pointer", "-g")), check=True)
        env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", OMP_NUM_THREADS="4",
                   ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:abort_on_error=0",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
        res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=900)
        assert res.returncode == 0 and "pins ok" in res.stdout, res.stderr[-4000:]
        assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-4000:]
