"""Pins of the oracle's tree rule for candidates drawn from the draft (recursive rejection).

* Exhaustive, over several rounds: with a context-dependent target and draft model on V <= 3 and
  fixed tree shapes (two or three children at the root, grandchildren, a chain), every assignment of
  candidate tokens is weighted by the probability of drawing it (each child independently from its
  parent's draft row), every way the uniforms can fall by its cell length (the oracle is checked to
  flip at its reported ratios and to draw at the CDF interval midpoints); the joint law of the first
  H committed tokens must equal the target's (lossless decoding).
* A chain of single children is the linear rule: same ratios, accepted lengths and tokens as the
  linear verify on the same rows and uniforms.
* Draft rows equal to the target rows accept the first child at every node.
* A candidate the draft cannot draw (zero draft probability under the nucleus) sets Q_ZERO.

The rule restated ([alphalab] "Linear 與 Tree sampler" leaves the candidate rule open): child i of
v is kept with probability min(1, r_{i-1}(x_i) / q_v(x_i)), r_0 = p_v; a rejection replaces the
residual by max(0, r_{i-1} - q_v) renormalised; with no child kept one token is drawn from the last
residual.
"""
import itertools

import numpy as np
import pytest

from refdist import ref_probs
from test_oracle_exhaustive import (_ar_joint, _check_cdf_midpoints, _multi_round_law,
                                    _table_model)

TOL = 1e-12


def sampled_tree_outcomes(orc, p, q, parent, tokens, T, max_depth):
    """Exact outcome law of one sampled-tree verify: [(prob, committed tuple)]."""
    N = len(parent)
    P_, Q_ = p[None], q[None]
    par = np.array([parent], np.int32)
    tok = np.array([tokens], np.int32)

    def verify(ua, ur, want=False):
        return orc.verify_tree_sampled(P_, Q_, par, tok, max_depth, T=T, u_accept=ua,
                                       u_resample=ur, want_resid=want)
    ratio = verify(np.zeros((1, N)), np.zeros(1))["node_ratios"][0]
    children = {v: [c for c in range(N) if parent[c] == v] for v in range(-1, N)}
    outs = []

    def walk(v, prob, path, rejected):
        rej = 1.0
        ch = children[v]
        for i, c in enumerate(ch):
            pa = prob * rej * ratio[c]
            if pa > 0.0:
                walk(c, pa, path + [c], rejected + ch[:i])
            rej *= (1.0 - ratio[c])
        pstop = prob * rej
        if pstop <= 0.0:
            return
        ua = np.zeros((1, N))
        for n in rejected + ch:
            ua[0, n] = ratio[n]  # u == ratio rejects (strict test)
        o = verify(ua, np.array([0.5]), True)
        assert o["accept_len"][0] == len(path)
        assert list(o["accept_nodes"][0, :len(path)]) == path
        w, S = o["resid_w"][0], o["resid_S"][0]
        _check_cdf_midpoints(orc, lambda u: verify(ua, np.array([u])), w, S,
                             lambda oo: int(oo["out_tokens"][0, len(path)]))
        committed = tuple(tokens[n] for n in path)
        for x in range(len(w)):
            if w[x] > 0:
                outs.append((pstop * w[x] / S, committed + (x,)))

    walk(-1, 1.0, [], [])
    return outs


def _node_paths(parent, tokens):
    paths = []
    for j, v in enumerate(parent):
        paths.append((paths[v] if v >= 0 else []) + [tokens[j]])
    return paths


def _sampled_round(orc, ar, dr, prefix, V, parent, T, depth):
    """Outcome law of one round: candidates drawn from the draft model for a fixed tree shape."""
    N = len(parent)
    res = {}
    for toks in itertools.product(range(V), repeat=N):
        paths = _node_paths(parent, list(toks))
        P = 1.0
        for j, v in enumerate(parent):
            ctx = list(prefix) + (paths[v] if v >= 0 else [])
            P *= ref_probs(dr(ctx), T)[toks[j]]
        if P == 0.0:
            continue
        p = np.stack([ar(list(prefix))] + [ar(list(prefix) + pth) for pth in paths])
        q = np.stack([dr(list(prefix))] + [dr(list(prefix) + pth) for pth in paths])
        for prob, ext in sampled_tree_outcomes(orc, p, q, parent, list(toks), T, depth):
            res[ext] = res.get(ext, 0.0) + P * prob
    return res


@pytest.mark.parametrize("V,parent,H,T", [
    (3, [-1, -1], 3, 1.0),              # two candidates at the root
    (3, [-1, -1, -1], 3, 0.8),          # three candidates, duplicates common
    (3, [-1, -1, 0, 1], 3, 1.0),        # two children, one grandchild each
    (2, [-1, 0, 1], 4, 1.0),            # a chain
    (3, [-1, -1, 0, 0], 3, 1.2),        # two root candidates, the first with two children
])
def test_sampled_tree_multi_round_lossless(orc, V, parent, H, T):
    depth = 1
    for j, v in enumerate(parent):
        d = 1
        while v >= 0:
            d += 1
            v = parent[v]
        depth = max(depth, d)
    ar = _table_model(55, V, 1.5)
    dr = _table_model(66, V, 1.5)
    got = _multi_round_law(lambda pre: _sampled_round(orc, ar, dr, pre, V, parent, T, depth), H)
    want = _ar_joint(ar, V, H, T)
    assert abs(sum(got.values()) - 1.0) < TOL
    for seq, pr in want.items():
        assert abs(got.get(seq, 0.0) - pr) < TOL, seq


@pytest.mark.parametrize("seed", range(4))
def test_chain_equals_linear(orc, seed):
    rng = np.random.default_rng(seed)
    V, B = 50, 5
    p = (rng.standard_normal((B + 1, V)) * 2).astype(np.float32)
    q = (p + rng.standard_normal((B + 1, V))).astype(np.float32)
    d = rng.integers(0, V, size=B).astype(np.int32)
    parent = np.arange(-1, B - 1, dtype=np.int32)
    for trial in range(6):
        ua = rng.random((1, B))
        ur = rng.random(1)
        tr = orc.verify_tree_sampled(p[None], q[None], parent[None], d[None], B, u_accept=ua,
                                     u_resample=ur)
        li = orc.verify_linear(p[None], q[None, :B], d[None], u_accept=ua, u_resample=ur)
        assert np.allclose(tr["node_ratios"][0], li["ratios"][0], rtol=0, atol=1e-15)
        k = li["accept_len"][0]
        assert tr["accept_len"][0] == k
        assert (tr["out_tokens"][0, :k + 1] == li["out_tokens"][0, :k + 1]).all()


def test_equal_draft_accepts_first_child(orc):
    rng = np.random.default_rng(7)
    V = 40
    parent = np.array([[-1, -1, 0, 0, 2]], np.int32)
    toks = rng.integers(0, V, size=(1, 5)).astype(np.int32)
    p = (rng.standard_normal((1, 6, V)) * 2).astype(np.float32)
    for step in range(10):
        o = orc.verify_tree_sampled(p, p, parent, toks, 3, seed=9, step=step)
        assert o["accept_len"][0] == 3 and list(o["accept_nodes"][0]) == [0, 2, 4]
        assert (o["node_ratios"][0, [0, 2, 4]] == 1.0).all()


def test_undrawable_candidate_sets_q_zero(orc):
    V = 10
    p = np.zeros((1, 3, V), np.float32)
    q = np.zeros((1, 3, V), np.float32)
    q[0, 0, 5] = 20.0  # the root's draft nucleus at top_p 0.5 is token 5 alone
    parent = np.array([[-1, -1]], np.int32)
    toks = np.array([[5, 2]], np.int32)
    o = orc.verify_tree_sampled(p, q, parent, toks, 1, top_p=0.5)
    assert o["status"][0] & orc.ST_Q_ZERO
