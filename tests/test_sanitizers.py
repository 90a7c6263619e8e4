"""The oracle and the C ABI's host code under AddressSanitizer and UBSan (CPU only).

The oracle is rebuilt with gcc -fsanitize=address,undefined and every pin runs against
it in a child process with gcc's ASan runtime preloaded; a copy of the oracle with one
planted heap overflow shows that the sanitizer is live in that set-up.  The library's
host code (argument validation, error text, pair counts, launch set-up) is rebuilt by
hipcc with the sanitizers on the host side only, and the ABI tests run against it in a
child process with clang's runtime preloaded.  No GPU is touched: every ABI test here
is rejected or answered on the host.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
SAN_FLAGS = ("-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-g")
ASAN_OPTIONS = "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0:abort_on_error=0"

PINS_SCRIPT = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {here!r})
from oracle import oracle
from oracle_pins import ALL_PINS
lib = oracle.load({lib!r}, build_if_missing=False)
for pin in ALL_PINS:
    pin(lib)
    print("pin ok", pin.__name__, flush=True)
print("ALL PINS RAN", flush=True)
"""


def _gcc_asan():
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's libasan.so is not installed")
    return path


def _run_pins(lib_path, preload):
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS=ASAN_OPTIONS,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    script = PINS_SCRIPT.format(root=ROOT, here=HERE, lib=lib_path)
    return subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env,
                          timeout=600)


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    preload = _gcc_asan()
    lib = oracle.build(out=str(tmp_path / "libts_oracle_san.so"), extra_flags=SAN_FLAGS)
    r = _run_pins(lib, preload)
    assert r.returncode == 0 and "ALL PINS RAN" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_sanitized_oracle_catches_a_planted_overflow(tmp_path):
    """The score buffer of the full routine (the first allocation of that form in the
    source) allocated one element short: the first row that sees every key of the
    longest sequence writes past it, and ASan must stop the run there."""
    preload = _gcc_asan()
    src = open(os.path.join(ROOT, "oracle", "ts_oracle.c")).read()
    site = "double* z = (double*)malloc(sizeof(double) * (size_t)max_len);"
    assert src.index(site) < src.index("int ts_oracle_prefill_rows(")
    planted = tmp_path / "planted.c"
    planted.write_text(src.replace(site, "double* z = (double*)malloc(sizeof(double) * (size_t)(max_len - 1));", 1))
    lib = oracle.build(src=str(planted), out=str(tmp_path / "libplanted.so"), extra_flags=SAN_FLAGS)
    r = _run_pins(lib, preload)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, (r.returncode, r.stderr[-2000:])


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    from sinks_ts_mha_amd import build
    lib = build.build_host_sanitized(str(tmp_path))
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the ABI layer is not instrumented"
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), ASAN_OPTIONS=ASAN_OPTIONS,
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", TS_MHA_LIBRARY=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_abi.py")], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "runtime error" not in r.stdout + r.stderr and "AddressSanitizer" not in r.stdout + r.stderr
