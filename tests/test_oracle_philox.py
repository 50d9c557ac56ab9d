"""Pins of the oracle's Philox4x32-10 and of its uniform mapping.

The oracle's Philox is checked against an independent implementation: rocRAND's philox4x32_10
engine, compiled here from its open header and run on the host (Salmon et al., SC'11, is the
published definition both follow)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    rng = np.random.default_rng(12345)
    cases = [(0, 0, 0, 0, 0), (1, 2, 3, 4, 5), (0xDEADBEEFDEADBEEF, 7, 0, 1, 199),
             (2**64 - 1, 0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF),
             (12345, 63, 15, 2, 9999)]
    for _ in range(200):
        cases.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                      int(rng.integers(0, 2**32)), int(rng.integers(0, 2**30)),
                      int(rng.integers(0, 2**32)), int(rng.integers(0, 2**32))))
    return cases


@pytest.fixture(scope="module")
def rocrand_ref():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("hipcc / rocRAND headers not available")
    d = tempfile.mkdtemp(prefix="philox_ref_")
    exe = os.path.join(d, "philox_ref")
    subprocess.check_call([hipcc, "-O1", "-o", exe, os.path.join(HERE, "philox_rocrand_ref.cpp")],
                          stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    yield exe
    shutil.rmtree(d, ignore_errors=True)


def test_philox_matches_rocrand(orc, rocrand_ref):
    cases = _cases()
    inp = "".join(f"{s} {a} {b} {c} {d}\n" for s, a, b, c, d in cases)
    out = subprocess.run([rocrand_ref], input=inp, capture_output=True, text=True, check=True).stdout
    ref = [tuple(int(x) for x in line.split()) for line in out.strip().splitlines()]
    assert len(ref) == len(cases)
    for (s, a, b, c, d), want in zip(cases, ref):
        got = tuple(int(x) for x in orc.philox(s, [a, b, c, d]))
        assert got == want, (s, a, b, c, d)


def test_uniform_is_top53_bits_of_words01(orc):
    for (s, req, pos, pur, step) in [(0, 0, 0, 0, 0), (99, 3, 7, 1, 12), (2**64 - 1, 5, 63, 2, 2**32 - 1)]:
        x = orc.philox(s, [req, pos, pur, step])
        bits = (int(x[0]) << 32) | int(x[1])
        want = (bits >> 11) / 2.0**53
        assert orc.uniform(s, req, pos, pur, step) == want


def test_uniform_range_and_moments(orc):
    u = np.array([orc.uniform(7, r, i, 0, 3) for r in range(2000) for i in range(8)])
    assert u.min() >= 0.0 and u.max() < 1.0
    n = u.size
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / n)
    # Kolmogorov-Smirnov against U(0,1) at a generous level
    from scipy import stats
    assert stats.kstest(u, "uniform").pvalue > 1e-4


def test_uniform_keys_are_distinct_streams(orc):
    # changing any key word changes the draw
    base = orc.uniform(5, 1, 2, 0, 3)
    for args in [(6, 1, 2, 0, 3), (5, 2, 2, 0, 3), (5, 1, 3, 0, 3), (5, 1, 2, 1, 3), (5, 1, 2, 0, 4)]:
        assert orc.uniform(*args) != base
