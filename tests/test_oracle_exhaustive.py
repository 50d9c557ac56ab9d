"""Exhaustive pins of the oracle's verify rule on tiny vocabularies.

The oracle is driven with explicit uniforms.  For every drafted block and every way the uniforms can
fall, the probability of each outcome is the length of the uniform cell that leads to it: an accept
test passes for u in [0, ratio) (the oracle is checked to flip exactly at its reported ratio), and
the final draw returns token x for u' in its CDF interval of width w_x / S (the oracle is checked to
return x at the interval midpoint).  Summing over all outcomes gives the exact law of what the oracle
commits, which must equal the target (AR) law computed from the logits by an independent softmax:

* per position for row-independent targets (the committed token at every reached position has law
  p_j; reaching j+1 has probability reach_j * sum_x min(p_j(x), q_j(x)) -- the acceptance rate of
  speculative sampling, the lineage the pages cite);
* jointly over several rounds for a context-dependent target and draft model (lossless decoding);
* the same for the tree rule, with trees built from a draft model;
* the tokens-per-forward bound 1 <= TPF <= (B+1)/2 in the Uno layout, where position 1 comes from
  the AR itself.

Source of the properties: [alphalab] "Uno Ψ-Spec 是什麼？…", §"Uno Ψ-Spec 怎麼運作？完整走一次四個 Token"
(keep the longest accepted prefix, residual draw at the first rejection, bonus on full accept, TPF
bound) and §"為什麼 lossless 不等於答案完全一樣？" (the output law equals the base AR's).
"""
import itertools

import numpy as np
import pytest

from refdist import bf16_round, bf16_value, ref_probs

TOL = 1e-12


def _check_cdf_midpoints(orc, call, w, S, want_fn):
    """The oracle's draw returns x for u' at the middle of x's CDF interval."""
    C = 0.0
    for x in range(len(w)):
        if w[x] > 0 and w[x] / S > 1e-9:
            mid = (C + w[x] / 2) / S
            assert want_fn(call(mid)) == x
        C += w[x]


def linear_outcomes(orc, p, q, T, top_p, flags, d):
    """Exact outcome law of one linear verify call for a fixed drafted block d.
    Returns (ratios, [(prob, k, committed_token, w, S)])."""
    B = len(d)
    dd = np.array([d], dtype=np.int32)
    base = orc.verify_linear(p[None], q[None], dd, T=T, top_p=top_p, flags=flags,
                             u_accept=np.zeros((1, B)), u_resample=np.zeros(1))
    rat = base["ratios"][0]
    outs = []
    P = 1.0
    for j in range(B + 1):
        if P == 0.0:
            break
        if j < B and rat[j] >= 1.0:
            P *= rat[j]
            continue
        ua = np.zeros((1, B))
        if j < B:
            ua[0, j] = rat[j]  # u == ratio must reject (strict test)
        o = orc.verify_linear(p[None], q[None], dd, T=T, top_p=top_p, flags=flags, u_accept=ua,
                              u_resample=np.array([0.5]), want_resid=True)
        assert o["accept_len"][0] == j
        if j < B and rat[j] > 0.0:
            ua2 = ua.copy()
            ua2[0, j] = np.nextafter(rat[j], 0.0)  # just below the ratio accepts
            o2 = orc.verify_linear(p[None], q[None], dd, T=T, top_p=top_p, flags=flags, u_accept=ua2,
                                   u_resample=np.array([0.5]))
            assert o2["accept_len"][0] > j
        w, S = o["resid_w"][0], o["resid_S"][0]
        pstop = P * ((1.0 - rat[j]) if j < B else 1.0)

        def call(u, ua=ua):
            return orc.verify_linear(p[None], q[None], dd, T=T, top_p=top_p, flags=flags,
                                     u_accept=ua, u_resample=np.array([u]))
        _check_cdf_midpoints(orc, call, w, S, lambda o: int(o["out_tokens"][0, j]))
        for x in range(len(w)):
            if w[x] > 0:
                outs.append((pstop * w[x] / S, j, x))
        if j < B:
            P *= rat[j]
    return rat, outs


def _make_rows(rng, n, V, dtype, ties):
    if ties:
        vals = rng.integers(-6, 7, size=(n, V)) * 0.5
    else:
        vals = rng.standard_normal((n, V)) * 1.5
    if dtype == "bf16":
        return bf16_round(vals)
    return vals.astype(np.float32)


def _values(rows):
    return bf16_value(rows) if rows.dtype == np.uint16 else rows.astype(np.float64)


CASES = [
    # (V, B, dtype, ties, T, top_p, uno)
    (2, 1, "f32", False, 1.0, 1.0, False),
    (3, 2, "f32", False, 1.0, 1.0, False),
    (5, 3, "f32", False, 0.7, 1.0, False),
    (8, 2, "bf16", True, 1.0, 1.0, False),
    (6, 3, "bf16", True, 1.3, 1.0, False),
    (5, 2, "f32", True, 1.0, 0.8, False),
    (6, 3, "bf16", True, 0.7, 0.9, False),
    (4, 3, "f32", False, 1.0, 1.0, True),
    (7, 2, "bf16", True, 0.9, 0.85, True),
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("seed", [0, 1])
def test_linear_law_equals_target(orc, case, seed):
    V, B, dtype, ties, T, top_p, uno = case
    rng = np.random.default_rng(1000 * seed + V * 10 + B)
    p = _make_rows(rng, B + 1, V, dtype, ties)
    q = _make_rows(rng, B, V, dtype, ties)
    flags = orc.FIRST_FROM_TARGET if uno else 0
    if uno:
        q[0] = p[0]  # position 1 is drawn from the AR itself
    pv, qv = _values(p), _values(q)
    pref = [ref_probs(pv[j], T, top_p) for j in range(B + 1)]
    qref = [ref_probs(qv[i], T, top_p) for i in range(B)]
    law = np.zeros((B + 1, V))
    for d in itertools.product(range(V), repeat=B):
        Pd = float(np.prod([qref[i][d[i]] for i in range(B)]))
        if Pd == 0.0:
            continue
        rat, outs = linear_outcomes(orc, p, q, T, top_p, flags, d)
        # accepted positions commit the drafted token
        P = Pd
        for j in range(B):
            law[j, d[j]] += P * rat[j]
            P *= rat[j]
        for prob, j, x in outs:
            law[j, x] += Pd * prob
    reach = law.sum(axis=1)
    assert abs(reach[0] - 1.0) < TOL
    for j in range(B + 1):
        assert np.max(np.abs(law[j] - reach[j] * pref[j])) < TOL, (j, law[j], reach[j] * pref[j])
    # acceptance rate of speculative sampling: P(reach j+1) = P(reach j) * sum_x min(p_j, q_j)
    for j in range(B):
        alpha = 1.0 if (uno and j == 0) else np.minimum(pref[j], qref[j]).sum()
        assert abs(reach[j + 1] - reach[j] * alpha) < TOL


def _table_model(seed, V, scale):
    cache = {}

    def logits(prefix):
        key = tuple(prefix)
        if key not in cache:
            h = abs(hash((seed,) + key)) % (2**32)
            cache[key] = (np.random.default_rng(h).standard_normal(V) * scale).astype(np.float32)
        return cache[key]
    return logits


def _ar_joint(ar, V, H, T):
    law = {}
    for seq in itertools.product(range(V), repeat=H):
        pr = 1.0
        for t in range(H):
            pr *= ref_probs(ar(seq[:t]), T)[seq[t]]
        law[seq] = pr
    return law


def _linear_round(orc, ar, dr, prefix, V, B, T, uno):
    """Outcome law of one verify round from `prefix`: {extension tuple: probability}."""
    res = {}
    for d in itertools.product(range(V), repeat=B):
        P = 1.0
        for i in range(B):
            ctx = list(prefix) + list(d[:i])
            src = ar if (uno and i == 0) else dr
            P *= ref_probs(src(ctx), T)[d[i]]
        if P == 0.0:
            continue
        p = np.stack([ar(list(prefix) + list(d[:j])) for j in range(B + 1)])
        q = np.stack([(ar if (uno and i == 0) else dr)(list(prefix) + list(d[:i])) for i in range(B)])
        flags = orc.FIRST_FROM_TARGET if uno else 0
        rat, outs = linear_outcomes(orc, p, q, T, 1.0, flags, d)
        for prob, k, x in outs:
            ext = tuple(d[:k]) + (x,)
            res[ext] = res.get(ext, 0.0) + P * prob
            if uno:
                assert 2 <= len(ext) <= B + 1, ext  # 1 <= TPF = committed / 2 <= (B+1)/2
    return res


def _multi_round_law(round_fn, H):
    """Distribution of the first H tokens after repeating rounds from the empty prefix."""
    done = {}
    todo = {(): 1.0}
    while todo:
        nxt = {}
        for prefix, pr in todo.items():
            for ext, pe in round_fn(prefix).items():
                s = prefix + ext
                if len(s) >= H:
                    done[s[:H]] = done.get(s[:H], 0.0) + pr * pe
                else:
                    nxt[s] = nxt.get(s, 0.0) + pr * pe
        todo = nxt
    return done


@pytest.mark.parametrize("V,B,H,T,uno", [(3, 2, 4, 1.0, False), (3, 3, 4, 0.8, True),
                                         (4, 2, 3, 1.0, True), (2, 3, 5, 1.0, False)])
def test_linear_multi_round_lossless(orc, V, B, H, T, uno):
    ar = _table_model(11, V, 1.5)
    dr = _table_model(22, V, 1.5)
    got = _multi_round_law(lambda pre: _linear_round(orc, ar, dr, pre, V, B, T, uno), H)
    want = _ar_joint(ar, V, H, T)
    assert abs(sum(got.values()) - 1.0) < TOL
    for seq, pr in want.items():
        assert abs(got.get(seq, 0.0) - pr) < TOL, seq


# ------------------------------------------------------------------------------------------------
# tree rule
# ------------------------------------------------------------------------------------------------
def tree_outcomes(orc, p, parent, tokens, T, top_p, max_depth):
    """Exact outcome law of one tree verify call: [(prob, committed tuple)]."""
    N = len(parent)
    P_ = p[None]
    par = np.array([parent], np.int32)
    tok = np.array([tokens], np.int32)
    base = orc.verify_tree(P_, par, tok, max_depth, T=T, top_p=top_p, u_accept=np.zeros((1, N)),
                           u_resample=np.zeros(1))
    ratio = base["node_ratios"][0]
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
            ua[0, n] = ratio[n]
        o = orc.verify_tree(P_, par, tok, max_depth, T=T, top_p=top_p, u_accept=ua,
                            u_resample=np.array([0.5]), want_resid=True)
        assert o["accept_len"][0] == len(path)
        assert list(o["accept_nodes"][0, :len(path)]) == path
        w, S = o["resid_w"][0], o["resid_S"][0]

        def call(u, ua=ua):
            return orc.verify_tree(P_, par, tok, max_depth, T=T, top_p=top_p, u_accept=ua,
                                   u_resample=np.array([u]))
        _check_cdf_midpoints(orc, call, w, S, lambda o: int(o["out_tokens"][0, len(path)]))
        committed = tuple(tokens[n] for n in path)
        for x in range(len(w)):
            if w[x] > 0:
                outs.append((pstop * w[x] / S, committed + (x,)))

    walk(-1, 1.0, [], [])
    return outs


def _draft_tree(dr, prefix, V, k, depth, T):
    """Prefix tree: each node proposes the top-k tokens of the draft model (ties: lower id)."""
    parent, tokens, paths = [], [], []

    def add(v, path, dep):
        if dep > depth:
            return
        pr = ref_probs(dr(list(prefix) + path), T)
        order = sorted(range(V), key=lambda t: (-pr[t], t))[:k]
        for t in order:
            parent.append(v)
            tokens.append(t)
            paths.append(path + [t])
    add(-1, [], 1)  # then breadth-first below the root's children
    j = 0
    while j < len(parent):
        dep = len(paths[j])
        if dep < depth:
            pr = ref_probs(dr(list(prefix) + paths[j]), T)
            order = sorted(range(V), key=lambda t: (-pr[t], t))[:k]
            for t in order:
                parent.append(j)
                tokens.append(t)
                paths.append(paths[j] + [t])
        j += 1
    return parent, tokens, paths


def _tree_round(orc, ar, dr, prefix, V, k, depth, T):
    parent, tokens, paths = _draft_tree(dr, prefix, V, k, depth, T)
    rows = [ar(list(prefix))] + [ar(list(prefix) + pth) for pth in paths]
    p = np.stack(rows)
    res = {}
    for prob, ext in tree_outcomes(orc, p, parent, tokens, T, 1.0, depth):
        res[ext] = res.get(ext, 0.0) + prob
    return res


@pytest.mark.parametrize("V,k,depth,H,T", [(3, 2, 2, 3, 1.0), (4, 2, 2, 3, 0.8), (3, 1, 3, 4, 1.0),
                                           (5, 3, 1, 2, 1.0)])
def test_tree_multi_round_lossless(orc, V, k, depth, H, T):
    ar = _table_model(33, V, 1.5)
    dr = _table_model(44, V, 1.5)
    got = _multi_round_law(lambda pre: _tree_round(orc, ar, dr, pre, V, k, depth, T), H)
    want = _ar_joint(ar, V, H, T)
    assert abs(sum(got.values()) - 1.0) < TOL
    for seq, pr in want.items():
        assert abs(got.get(seq, 0.0) - pr) < TOL, seq


@pytest.mark.parametrize("seed", range(6))
def test_tree_single_level_law_with_duplicate_and_topp(orc, seed):
    """One level, arbitrary (even duplicated) candidate tokens, with a nucleus: the committed
    first token has the law of the root row."""
    rng = np.random.default_rng(seed)
    V = 6
    nchild = 4
    parent = [-1] * nchild
    tokens = list(rng.integers(0, V, size=nchild))
    tokens[-1] = tokens[0]  # a duplicated sibling token must get ratio 0
    p = bf16_round(rng.integers(-4, 5, size=(nchild + 1, V)) * 0.5)
    top_p = [1.0, 0.9][seed % 2]
    outs = tree_outcomes(orc, p, parent, tokens, 1.0, top_p, 1)
    law = np.zeros(V)
    for prob, ext in outs:
        law[ext[0]] += prob
    want = ref_probs(bf16_value(p[0]), 1.0, top_p)
    assert np.max(np.abs(law - want)) < TOL
    o = orc.verify_tree(p[None], np.array([parent], np.int32), np.array([tokens], np.int32), 1,
                        top_p=top_p, u_accept=np.zeros((1, nchild)), u_resample=np.zeros(1))
    assert o["node_ratios"][0, -1] == 0.0


@pytest.mark.parametrize("seed", range(5))
def test_chain_tree_equals_linear_with_one_hot_drafts(orc, seed):
    """A chain tree is the linear rule with one-hot draft rows: same ratios, tokens, lengths."""
    rng = np.random.default_rng(50 + seed)
    V, B = 7, 4
    p = (rng.standard_normal((B + 1, V)) * 2).astype(np.float32)
    d = rng.integers(0, V, size=B).astype(np.int32)
    q = np.full((B, V), -np.inf, np.float32)
    q[np.arange(B), d] = 0.0
    parent = np.arange(-1, B - 1, dtype=np.int32)
    for trial in range(40):
        ua = rng.random((1, B))
        ur = rng.random(1)
        lin = orc.verify_linear(p[None], q[None], d[None], u_accept=ua, u_resample=ur)
        tr = orc.verify_tree(p[None], parent[None], d[None], B, u_accept=ua, u_resample=ur)
        assert np.array_equal(lin["ratios"][0], tr["node_ratios"][0])
        assert lin["accept_len"][0] == tr["accept_len"][0]
        assert np.array_equal(lin["out_tokens"][0], tr["out_tokens"][0])
