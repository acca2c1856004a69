"""CPU runs under AddressSanitizer and UndefinedBehaviorSanitizer.

* The C oracle (oracle/parallax_oracle.c), built by gcc with
  -fsanitize=address,undefined, runs every pin of tests/test_oracle_pins.py.
* The library's host code (argument checks, split and workspace policy),
  built by hipcc with the sanitizers on the host side only, runs the ABI
  tests of tests/test_abi.py that need no GPU: every rejection path, the
  size queries and the exported symbols.

Each run is a subprocess with the matching sanitizer runtime preloaded (the
Python interpreter itself is not instrumented).  Any sanitizer report aborts
the run (-fno-sanitize-recover=all), which fails the test.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV_BASE = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1", "UBSAN_OPTIONS": "print_stacktrace=1"}


def _run(code, preload, *args):
    env = dict(os.environ, **ENV_BASE, LD_PRELOAD=preload)
    return subprocess.run([sys.executable, "-c", code, *args], capture_output=True, text=True, timeout=600,
                          env=env, cwd=ROOT)


ORACLE_RUN = r"""
import sys
sys.path.insert(0, "tests")
sys.path.insert(0, ".")
import oracle
import test_oracle_pins as pins
lib = oracle.load_variant(sys.argv[1])
for pin in pins.PINS:
    pin(lib)
    print("ok", pin.__name__, flush=True)
print("all pins passed")
"""


def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    gcc_rt = [subprocess.run(["gcc", f"-print-file-name={n}"], capture_output=True, text=True).stdout.strip()
              for n in ("libasan.so", "libubsan.so")]
    if not all(os.path.isabs(p) and os.path.exists(p) for p in gcc_rt):
        pytest.skip("gcc sanitizer runtimes not installed")
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-o", so,
                    os.path.join(ROOT, "oracle", "parallax_oracle.c"), "-lm"], check=True)
    res = _run(ORACLE_RUN, " ".join(gcc_rt), so)
    print(res.stdout[-2000:], res.stderr[-4000:])
    assert res.returncode == 0 and "all pins passed" in res.stdout


ABI_RUN = r"""
import os, sys
sys.path.insert(0, ".")
from transformer_attention_flash_amd import _native as N
N.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", "tests/test_abi.py", "-k",
                      "not c_caller and not product_does_not_use"]))
"""


def test_host_checks_under_address_and_ub_sanitizers(tmp_path):
    from transformer_attention_flash_amd.build import build_library, sanitizer_runtime

    try:
        rt = sanitizer_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    so = build_library(lib_path=str(tmp_path / "libparallax_san.so"), host_sanitize=True)
    out = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert "__asan_" in out, "the host code is not instrumented"
    res = _run(ABI_RUN, rt, so)
    print(res.stdout[-3000:], res.stderr[-4000:])
    assert res.returncode == 0 and " passed" in res.stdout and "failed" not in res.stdout
