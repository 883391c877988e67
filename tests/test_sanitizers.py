"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: the oracle's pins and the C-ABI tests (argument
validation, planning, error reporting; no GPU) run again in a subprocess with
sanitized builds of both and the sanitizer runtime preloaded. Any report fails
the run."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.timeout(600)
def test_oracle_pins_and_abi_under_sanitizers():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("no sanitizer runtime next to gcc")
    sys.path.insert(0, ROOT)
    from lightning_indexer_top_idx_amd import build

    lib = build.build(sanitize=True)
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": f"{asan}:{ubsan}",
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1:protect_shadow_gap=0",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        "LIT_LIBRARY": lib,
        "ORACLE_SANITIZED": "1",
        "HIP_VISIBLE_DEVICES": "",  # host code only: never a launch on a real device
    })
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_abi.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=560)
    # -s: a sanitizer report goes to this process's stderr, not into a capture
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
