"""The CPU oracle and the seeded input generator under AddressSanitizer and
UndefinedBehaviorSanitizer: both C libraries are rebuilt instrumented and the oracle's pins run
against them in a child process (libasan preloaded, leaks not checked: the Python interpreter and
torch are not instrumented).  Any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _libasan():
    r = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(bool(os.environ.get("LD_PRELOAD")),
                    reason="another library is already preloaded in this environment")
def test_oracle_pins_clean_under_asan_and_ubsan():
    asan = _libasan()
    if asan is None:
        pytest.skip("gcc has no AddressSanitizer runtime here")
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    from fp4_block_scaled_amd import build as pb
    ref = ob.build(sanitize=True)
    syn = pb.build_synth(sanitize=True)
    env = dict(os.environ, LD_PRELOAD=asan, MXREF_LIB=ref, MXSYNTH_LIB=syn,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-s", "-p", "no:cacheprovider", "-x",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
