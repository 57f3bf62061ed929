"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only), with every oracle pin run against that build (CPU only).

The instrumented library is loaded into a child Python whose sanitizer
runtimes are preloaded (the interpreter itself is not instrumented).  A copy
of the oracle with one planted heap overflow is run the same way first, to
show that the sanitizer is live in that setting.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-std=c11", "-fopenmp", "-fPIC", "-shared"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _build(src_text, out_dir):
    c = os.path.join(out_dir, "orc_san.c")
    so = os.path.join(out_dir, "liborc_san.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc"] + SAN_FLAGS + [c, "-o", so, "-lm"])
    return so


def _run_pins(so, log_dir, extra=()):
    """Runs the pins against `so`; returns (exit code, pytest output, sanitizer
    reports).  The reports go to files under log_dir (pytest's own capture of
    the child's stderr would lose a report written as the process dies)."""
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    env = dict(os.environ, MOE_ORACLE_LIB=so, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=0:log_path={log_dir}/asan",
               UBSAN_OPTIONS=f"print_stacktrace=1:halt_on_error=1:log_path={log_dir}/ubsan")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", PINS]
                       + list(extra), env=env, capture_output=True, text=True, cwd=ROOT,
                       timeout=600)
    reports = ""
    for f in sorted(os.listdir(log_dir)):
        if f.startswith(("asan", "ubsan")):
            reports += open(os.path.join(log_dir, f)).read()
    return r.returncode, r.stdout + r.stderr, reports


@pytest.fixture(scope="module")
def sanitizers():
    if not (_runtime("libasan.so") and _runtime("libubsan.so")):
        pytest.skip("gcc sanitizer runtimes not installed")


def test_sanitizer_catches_a_planted_overflow(sanitizers, tmp_path):
    src = open(SRC).read()
    old = "double *p = malloc(sizeof(double) * (size_t)E);"
    assert old in src, "planting site moved; update this test"
    so = _build(src.replace(old, "double *p = malloc(sizeof(double) * (size_t)(E - 1));"), str(tmp_path))
    rc, _, reports = _run_pins(so, str(tmp_path), ["-k", "test_route_ids_match_brute_force"])
    assert rc != 0
    assert "AddressSanitizer: heap-buffer-overflow" in reports and "orc_route" in reports


def test_oracle_pins_clean_under_asan_ubsan(sanitizers, tmp_path):
    so = _build(open(SRC).read(), str(tmp_path))
    rc, out, reports = _run_pins(so, str(tmp_path))
    assert rc == 0, out[-3000:] + reports[-3000:]
    assert reports == "", reports[-3000:]
    assert " passed" in out
