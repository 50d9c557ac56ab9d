"""The B=4 walkthrough of the pages, pinned structurally (the page prints no numbers), plus
boundary pins of the rule.

Fixture: tests/golden/walkthrough_b4.json ([alphalab] "Uno Ψ-Spec 是什麼？…",
§"Uno Ψ-Spec 怎麼運作？完整走一次四個 Token")."""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

HERE = os.path.dirname(os.path.abspath(__file__))
FIX = json.load(open(os.path.join(HERE, "golden", "walkthrough_b4.json")))
B = FIX["block_size"]


def _rows(seed, V=64):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal((B + 1, V)) * 2).astype(np.float32)
    q = (p[:B] + rng.standard_normal((B, V)) * 1.5).astype(np.float32)
    return p, q, rng


@pytest.mark.parametrize("use_flag", [False, True])
def test_first_position_from_ar_always_accepted(orc, use_flag):
    assert FIX["first_position_from_ar_always_accepted"]
    p, q, rng = _rows(1)
    q[0] = p[0]  # T1 is the AR's own sample
    flags = orc.FIRST_FROM_TARGET if use_flag else 0
    for step in range(300):
        d = rng.integers(0, p.shape[1], size=(1, B)).astype(np.int32)
        o = orc.verify_linear(p[None], q[None], d, seed=77, step=step, flags=flags)
        assert o["accept_len"][0] >= 1
        assert o["out_tokens"][0, 0] == d[0, 0]
        assert o["ratios"][0, 0] == 1.0


def test_reject_at_third_discards_the_rest(orc):
    sc = FIX["scenarios"][0]
    rej = sc["rejected_position"] - 1
    p, q, rng = _rows(2)
    V = p.shape[1]
    for i in range(rej):
        q[i] = p[i]  # positions before the rejection pass for sure (ratio 1)
    for step in range(200):
        d = rng.integers(0, V, size=(1, B)).astype(np.int32)
        pp = p.copy()
        pp[rej, d[0, rej]] = -np.inf  # the AR gives the third draft zero probability
        o = orc.verify_linear(pp[None], q[None], d, seed=5, step=step)
        assert o["accept_len"][0] == rej
        out = o["out_tokens"][0]
        assert list(out[:rej]) == list(d[0, :rej])
        assert out[rej] != d[0, rej] and 0 <= out[rej] < V  # correction token
        assert all(out[i] == -1 for i in range(rej + 1, B + 1))  # discarded
        assert len(sc["committed"]) == rej + 1


def test_full_accept_gives_bonus_from_block_end_row(orc):
    sc = FIX["scenarios"][1]
    p, q, rng = _rows(3)
    V = p.shape[1]
    q[:] = p[:B]  # every draft passes
    seed = 9
    for step in range(200):
        d = rng.integers(0, V, size=(1, B)).astype(np.int32)
        o = orc.verify_linear(p[None], q[None], d, seed=seed, step=step)
        assert o["accept_len"][0] == B
        out = o["out_tokens"][0]
        assert list(out[:B]) == list(d[0]) and len(sc["committed"]) == B + 1
        # bonus = inverse CDF of the block-end row at the RESAMPLE uniform (independent routine)
        u = orc.uniform(seed, 0, B, orc.PURPOSE_RESAMPLE, step)
        pr = softmax(p[B].astype(np.float64))
        cdf = np.cumsum(pr)
        want = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
        assert out[B] == want


def test_tokens_per_forward_bound_in_uno_layout(orc):
    tpf = FIX["tokens_per_forward"]
    p, q, rng = _rows(4)
    q[0] = p[0]
    lo, hi = tpf["min"], (B + 1) / 2
    seen = set()
    for step in range(400):
        d = rng.integers(0, p.shape[1], size=(1, B)).astype(np.int32)
        d[0, 1:] = np.argsort(-q[1:], axis=1)[:, 0]  # likely drafts so long accepts occur
        o = orc.verify_linear(p[None], q[None], d, seed=11, step=step, flags=orc.FIRST_FROM_TARGET)
        committed = int(o["accept_len"][0]) + 1
        t = committed / tpf["forwards_per_round"]
        assert lo <= t <= hi
        seen.add(committed)
    assert min(seen) >= 2


def test_zero_weight_token_never_drawn(orc):
    """c = min{x : C_x > v} with a strict '>': at u' = 0 the first token of positive weight."""
    rng = np.random.default_rng(5)
    V = 12
    for trial in range(50):
        p = (rng.standard_normal((2, V)) * 2).astype(np.float32)
        p[:, :3] = -np.inf  # leading zero-weight tokens
        q = (rng.standard_normal((1, V)) * 2).astype(np.float32)
        d = np.array([[int(rng.integers(3, V))]], np.int32)
        for ua in [0.999999, 0.0]:
            o = orc.verify_linear(p[None], q[None], d, u_accept=np.array([[ua]]),
                                  u_resample=np.array([0.0]), want_resid=True)
            w = o["resid_w"][0]
            k = o["accept_len"][0]
            tok = o["out_tokens"][0, k]
            assert w[tok] > 0 and np.all(w[:tok] == 0)


def test_nucleus_boundary_is_inclusive(orc):
    """top_p equal to the largest probability keeps exactly that token ('mass >= top_p')."""
    rng = np.random.default_rng(6)
    for trial in range(20):
        l = (rng.standard_normal(30) * 2).astype(np.float32)
        pi, _, _ = orc.row_probs(l)
        top = float(pi.max())
        kept, _, margin = orc.row_probs(l, top_p=top)
        assert kept[int(np.argmax(l))] == 1.0 and np.count_nonzero(kept) == 1
        assert margin == 0.0


def test_status_bits(orc):
    p, q, _ = _rows(7, V=16)
    d = np.array([[1, 2, 3, 99]], np.int32)  # token 99 outside V
    o = orc.verify_linear(p[None], q[None], d, seed=1)
    assert o["status"][0] & orc.ST_BAD_TOKEN
    assert o["ratios"][0, 3] == 0.0
    pn = p.copy()
    pn[1, 4] = np.nan
    o = orc.verify_linear(pn[None], q[None], np.array([[1, 2, 3, 4]], np.int32), seed=1)
    assert o["status"][0] & orc.ST_NONFINITE
    qz = q.copy()
    qz[2, 3] = -np.inf  # drafted token with zero draft probability
    o = orc.verify_linear(p[None], qz[None], np.array([[1, 2, 3, 4]], np.int32), seed=1)
    assert o["status"][0] & orc.ST_Q_ZERO and o["ratios"][0, 2] == 1.0
    # tree: parent must precede its child
    pt = (np.random.default_rng(0).standard_normal((1, 3, 8))).astype(np.float32)
    o = orc.verify_tree(pt, np.array([[1, -1]], np.int32), np.array([[0, 1]], np.int32), 2, seed=1)
    assert o["status"][0] & orc.ST_BAD_PARENT


def test_argument_errors(orc):
    p, q, _ = _rows(8, V=8)
    d = np.zeros((1, B), np.int32)
    for kw in [dict(T=0.0), dict(T=float("nan")), dict(top_p=0.0), dict(top_p=1.5)]:
        with pytest.raises(ValueError):
            orc.verify_linear(p[None], q[None], d, **kw)
