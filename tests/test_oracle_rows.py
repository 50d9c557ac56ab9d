"""Pins of the oracle's row transform: temperature softmax and the tie-inclusive nucleus.

Closed forms (uniform row, two-token logistic), an independent library routine (scipy's softmax),
exact bf16 widening of known bit patterns, and a brute force over every subset for the nucleus."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax


def _bf16(values):
    """Round-to-nearest-even float32 -> bf16 bit patterns (exact for the values used here)."""
    f = np.asarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def test_constant_row_is_uniform(orc):
    for V in [1, 2, 7, 32, 1000]:
        for T in [0.3, 1.0, 2.5]:
            pi, st, _ = orc.row_probs(np.full(V, 3.25, np.float32), T=T)
            assert st == 0
            assert np.all(pi == 1.0 / V) or np.allclose(pi, 1.0 / V, rtol=0, atol=1e-16)


@pytest.mark.parametrize("T", [0.5, 0.7, 1.0, 3.0])
def test_two_tokens_logistic(orc, T):
    for a, b in [(0.0, 1.0), (-2.5, 4.0), (10.0, -10.0), (1e-3, 0.0)]:
        pi, st, _ = orc.row_probs(np.array([a, b], np.float32), T=T)
        a64, b64 = float(np.float32(a)), float(np.float32(b))
        want0 = 1.0 / (1.0 + math.exp((b64 - a64) / T))
        assert abs(pi[0] - want0) < 1e-15 and abs(pi[1] - (1 - want0)) < 1e-15


@pytest.mark.parametrize("T", [0.7, 1.0, 1.9])
def test_matches_scipy_softmax(orc, T):
    rng = np.random.default_rng(3)
    for V in [5, 64, 4099]:
        l = (rng.standard_normal(V) * 3).astype(np.float32)
        pi, st, _ = orc.row_probs(l, T=T)
        want = softmax(l.astype(np.float64) / T)
        # different summation order: agreement to a few ulps, relative
        assert np.max(np.abs(pi - want) / want) < 1e-13
        assert abs(pi.sum() - 1) < 1e-12


def test_bf16_widening_exact(orc):
    # 0x3F80 = 1.0, 0x4000 = 2.0, 0xC040 = -3.0, 0x3F00 = 0.5 ; row [1, 2, -3, 0.5]
    bits = np.array([0x3F80, 0x4000, 0xC040, 0x3F00], dtype=np.uint16)
    pi, st, _ = orc.row_probs(bits)
    want = softmax(np.array([1.0, 2.0, -3.0, 0.5]))
    assert np.max(np.abs(pi - want)) < 1e-15
    # same values as float32 give bit-identical probabilities
    pi32, _, _ = orc.row_probs(np.array([1.0, 2.0, -3.0, 0.5], np.float32))
    assert np.array_equal(pi, pi32)


def test_minus_inf_is_zero_mass_and_nonfinite_flags(orc):
    ninf = np.uint16(0xFF80)
    bits = np.array([0x3F80, ninf, 0x4000], dtype=np.uint16)
    pi, st, _ = orc.row_probs(bits)
    assert st == 0 and pi[1] == 0.0
    assert abs(pi[0] - 1 / (1 + math.e)) < 1e-15
    for bad in [np.array([0.0, np.nan], np.float32), np.array([0.0, np.inf], np.float32),
                np.array([-np.inf, -np.inf], np.float32)]:
        pi, st, _ = orc.row_probs(bad)
        assert st == orc.ST_NONFINITE and np.all(pi == 0)


def _nucleus_brute(pi, logits, top_p):
    """Smallest-cardinality set reaching top_p, closed upward under 'logit >=' (ties kept)."""
    V = len(pi)
    best = None
    for n in range(1, V + 1):
        for S in itertools.combinations(range(V), n):
            if sum(pi[list(S)]) >= top_p:
                lo = min(logits[list(S)])
                cand = frozenset(x for x in range(V) if logits[x] >= lo)
                if best is None or sum(pi[list(cand)]) < sum(pi[list(best)]) - 1e-300:
                    best = cand
        if best is not None:
            return best
    return frozenset(range(V))


@pytest.mark.parametrize("seed", range(40))
def test_nucleus_brute_force(orc, seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(1, 9))
    # coarse grid so equal logits (tie groups) are common
    l = (rng.integers(-4, 5, size=V) * 0.75).astype(np.float32)
    T = float(rng.choice([0.5, 1.0, 2.0]))
    top_p = float(rng.choice([0.05, 0.3, 0.5, 0.77, 0.9, 0.99]))
    base, _, _ = orc.row_probs(l, T=T)
    keep = _nucleus_brute(base, l.astype(np.float64), top_p)
    pi, st, margin = orc.row_probs(l, T=T, top_p=top_p)
    assert st == 0
    for x in range(V):
        if x in keep:
            want = base[x] / sum(base[list(keep)])
            assert abs(pi[x] - want) < 1e-15
        else:
            assert pi[x] == 0.0
    # margin: distance of top_p to the running masses around the boundary group
    kept_mass = sum(base[list(keep)])
    lo = min(l[list(keep)])
    above = sum(base[x] for x in range(V) if l[x] > lo)
    assert abs(margin - min(top_p - above, kept_mass - top_p)) < 1e-12


def test_nucleus_special_cases(orc):
    rng = np.random.default_rng(9)
    l = (rng.standard_normal(50) * 2).astype(np.float32)
    full, _, _ = orc.row_probs(l)
    same, _, _ = orc.row_probs(l, top_p=1.0)
    assert np.array_equal(full, same)
    # tiny top_p keeps exactly the argmax tie group
    l2 = l.copy()
    l2[[3, 17]] = l.max() + 1.0
    tiny, _, _ = orc.row_probs(l2, top_p=1e-9)
    assert tiny[3] == 0.5 and tiny[17] == 0.5 and tiny.sum() == 1.0
