"""The oracle built with the address and undefined-behaviour sanitizers (host code only) runs the
oracle's own pin tests in a child process; any out-of-bounds access, use after free or undefined
operation in the C oracle aborts that process with a report."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = ["test_oracle_rows.py", "test_oracle_exhaustive.py", "test_oracle_worked_example.py",
         "test_oracle_drafts.py", "test_oracle_tree_sampled.py", "test_oracle_kv.py",
         "test_oracle_lmhead.py", "test_oracle_stats.py"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    flags = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]
    so = oracle.build(force=True, out=str(tmp_path / "libpsispec_oracle_san.so"), checks=tuple(flags))
    env = dict(os.environ)
    env["PSISPEC_ORACLE_LIB"] = so
    env["LD_PRELOAD"] = f"{asan}:{ubsan}"
    # Python itself keeps memory until exit: leak reports would be about the interpreter
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *[os.path.join(ROOT, "tests", t) for t in TESTS]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
