"""The C oracle's own pins, run once more against a build of bt_oracle.c with
the address and undefined-behaviour sanitizers (host code only, on the CPU):
an out-of-bounds access, a signed overflow or an out-of-range float-to-int
conversion anywhere in the oracle aborts the run."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="no address-sanitizer runtime")
def test_oracle_pins_under_sanitizers(tmp_path):
    so = oracle.build_sanitized(str(tmp_path / "liboracle_sanitized.so"))
    env = dict(os.environ)
    env.update({
        oracle.LIB_ENV: so,
        "LD_PRELOAD": _runtime("libasan.so"),
        # Python itself is not built with the sanitizer: leaks at exit are its
        # own, so only memory errors and undefined behaviour are reported.
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "OMP_NUM_THREADS": "4",
    })
    tests = ["tests/test_oracle_pack.py", "tests/test_oracle_quant.py",
             "tests/test_oracle_matmul.py"]
    # -s: a sanitizer report goes to stderr just before the process ends
    r = subprocess.run([sys.executable, "-m", "pytest", "-s", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert " passed" in r.stdout
