"""Pins of the oracle's drafting step ([alphalab] walkthrough steps 1-2: the AR path samples the first
token of the block, the diffusion path proposes the rest; each drafted token is one inverse-CDF draw
from its row after temperature and the nucleus).

What pins it, independently of the oracle's own code:
  - equal logits over V = 32 (a power of two, so every prefix sum (x+1)/32 is exact): the draw at u
    is floor(32 u), the closed form of the inverse CDF with a strict '>';
  - u = 0 gives the first token of positive weight and u = 1 - 2^-53 the last one;
  - a row with one finite logit always gives that token;
  - the row layout: FIRST_FROM_TARGET takes position 0 from the AR row (any row stride), q row 0 is
    then never read (NaN there flags nothing), without the flag q row 0 is used;
  - scaling the logits by 1/T (a power of two, exact in fp64) equals the temperature T;
  - the Philox key: explicit uniforms equal to the uniform at (request, i, DRAFT, step) reproduce
    the default draw;
  - frequencies over many Philox draws match softmax(l / T) (chi-square), and with top-p every draw
    falls in the brute-force nucleus and frequencies match the renormalised nucleus;
  - a multi-round loop (draft, verify, commit) over a tabulated Markov AR at V = 6 in the Uno layout
    produces a token sequence whose transition frequencies match the AR's table (lossless across
    rounds), with 2 <= committed tokens per round <= B + 1.
"""
import numpy as np
import pytest
from scipy import stats

from refdist import nucleus_set, ref_probs


def _chisq(counts, probs):
    n = counts.sum()
    exp = n * probs
    big = exp >= 5.0
    obs_b = np.append(counts[big], counts[~big].sum())
    exp_b = np.append(exp[big], exp[~big].sum())
    if exp_b[-1] < 5.0:
        obs_b[-2] += obs_b[-1]
        exp_b[-2] += exp_b[-1]
        obs_b, exp_b = obs_b[:-1], exp_b[:-1]
    if len(obs_b) < 2:  # one outcome carries all the mass: every draw must be it
        return 1.0 if np.allclose(obs_b, exp_b) else 0.0
    return stats.chisquare(obs_b, exp_b).pvalue


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_equal_logits_closed_form(orc, T):
    V, n = 32, 400
    q = np.zeros((n, 1, V), np.float32)
    u = np.random.default_rng(3).random((n, 1))
    u[:64, 0] = np.arange(64) / 64.0  # also every breakpoint exactly and the midpoints
    o = orc.sample_drafts(None, q, T=T, u_draw=u)
    assert (o["tokens"][:, 0] == np.floor(32 * u[:, 0]).astype(np.int32)).all()
    assert (o["status"] == 0).all()


def test_first_and_last_positive_token(orc):
    V = 40
    row = np.full(V, -np.inf, np.float32)
    row[[5, 9, 30]] = [0.3, -1.0, 2.0]
    q = np.stack([row, row])[None]
    u = np.array([[0.0, 1.0 - 2.0**-53]])
    o = orc.sample_drafts(None, q, u_draw=u)
    assert o["tokens"].tolist() == [[5, 30]]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_finite_logit(orc, dtype):
    V, batch, B = 50, 4, 3
    rng = np.random.default_rng(5)
    hot = rng.integers(0, V, size=(batch, B))
    q = np.full((batch, B, V), -np.inf, np.float32)
    for r in range(batch):
        for i in range(B):
            q[r, i, hot[r, i]] = rng.normal() * 3
    if dtype == "bf16":
        q = (q.view(np.uint32) >> 16).astype(np.uint16)
    for step in range(5):
        o = orc.sample_drafts(None, q, seed=11, step=step)
        assert (o["tokens"] == hot).all()


def test_first_from_target_layout(orc):
    V, batch, B = 24, 3, 4
    rng = np.random.default_rng(9)
    ar_tok = rng.integers(0, V, size=batch)
    q_tok = rng.integers(0, V, size=(batch, B))
    q = np.full((batch, B, V), -np.inf, np.float32)
    for r in range(batch):
        for i in range(B):
            q[r, i, q_tok[r, i]] = 1.0
    # AR rows in the verify layout [batch][B+1][V]: only row 0 of each request is read
    ar = np.full((batch, B + 1, V), np.nan, np.float32)
    ar[:, 0, :] = -np.inf
    ar[np.arange(batch), 0, ar_tok] = 0.0
    qn = q.copy()
    qn[:, 0, :] = np.nan  # q row 0 is not read in this layout
    o = orc.sample_drafts(ar, qn, seed=2, flags=orc.FIRST_FROM_TARGET)
    assert (o["tokens"][:, 0] == ar_tok).all()
    assert (o["tokens"][:, 1:] == q_tok[:, 1:]).all()
    assert (o["status"] == 0).all()
    # packed [batch][V] AR rows give the same
    o2 = orc.sample_drafts(np.ascontiguousarray(ar[:, 0, :]), qn, seed=2,
                           flags=orc.FIRST_FROM_TARGET)
    assert (o2["tokens"] == o["tokens"]).all()
    # without the flag position 0 comes from q row 0
    o3 = orc.sample_drafts(None, q, seed=2)
    assert (o3["tokens"] == q_tok).all()
    o4 = orc.sample_drafts(None, qn, seed=2)
    assert (o4["status"][:, 0] == orc.ST_NONFINITE).all() and (o4["status"][:, 1:] == 0).all()


def test_temperature_is_logit_scaling(orc):
    V, batch, B = 300, 4, 5
    rng = np.random.default_rng(13)
    l = rng.normal(size=(batch, B, V)) * 3.0
    for T in (0.25, 2.0, 0.5):
        a = orc.sample_drafts(None, l, T=T, seed=77, step=3)
        b = orc.sample_drafts(None, l / T, T=1.0, seed=77, step=3)
        assert (a["tokens"] == b["tokens"]).all()


def test_philox_key_of_draft_draws(orc):
    V, batch, B = 64, 5, 4
    rng = np.random.default_rng(21)
    q = (rng.normal(size=(batch, B, V)) * 2).astype(np.float32)
    seed, step, base = 0xDEADBEEF12345, 7, 100
    u = np.array([[orc.uniform(seed, base + r, i, orc.PURPOSE_DRAFT, step) for i in range(B)]
                  for r in range(batch)])
    a = orc.sample_drafts(None, q, seed=seed, step=step, request_base=base)
    b = orc.sample_drafts(None, q, u_draw=u)
    assert (a["tokens"] == b["tokens"]).all()
    # the accept and resample purposes of the same counter give other uniforms
    ua = np.array([[orc.uniform(seed, base + r, i, orc.PURPOSE_ACCEPT, step) for i in range(B)]
                   for r in range(batch)])
    assert not np.array_equal(ua, u)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_frequencies_match_softmax(orc, T):
    V, reps, steps = 12, 2000, 10
    l = np.random.default_rng(31).normal(size=V) * 2.0
    q = np.broadcast_to(l.astype(np.float32), (reps, 1, V)).copy()
    counts = np.zeros(V)
    for s in range(steps):
        o = orc.sample_drafts(None, q, T=T, seed=5, step=s)
        counts += np.bincount(o["tokens"][:, 0], minlength=V)
    assert _chisq(counts, ref_probs(l.astype(np.float32), T)) > 1e-4


@pytest.mark.parametrize("top_p", [0.5, 0.8, 0.95])
def test_top_p_draws_stay_in_brute_force_nucleus(orc, top_p):
    V, reps, steps = 8, 1500, 8
    l = np.random.default_rng(int(top_p * 100)).normal(size=V).astype(np.float32) * 1.5
    T = 0.9
    pi = ref_probs(l, T)
    keep = nucleus_set(pi, l.astype(np.float64), top_p)
    q = np.broadcast_to(l, (reps, 1, V)).copy()
    counts = np.zeros(V)
    for s in range(steps):
        o = orc.sample_drafts(None, q, T=T, top_p=top_p, seed=8, step=s)
        counts += np.bincount(o["tokens"][:, 0], minlength=V)
    assert set(np.nonzero(counts)[0].tolist()) <= set(keep)
    assert _chisq(counts, ref_probs(l, T, top_p)) > 1e-4


def test_multi_round_loop_is_lossless(orc):
    """Uno-layout rounds over a Markov AR: p(next | last token) = softmax(A[last]); the drafts of
    positions 1..B-1 come from q rows that depend on the context only (parallel drafting).  The
    verify rows are the AR's rows at every drafted prefix.  Committed transitions must follow A."""
    V, B, chains, rounds = 6, 4, 64, 120
    rng = np.random.default_rng(41)
    A = rng.normal(size=(V, V)) * 1.5           # AR logits, row = previous token
    Q = A[None] + rng.normal(size=(B, V, V))    # draft logits of position i given the context
    ctx = rng.integers(0, V, size=chains)
    trans = np.zeros((V, V))
    committed_counts = []
    for step in range(rounds):
        ar = A[ctx].astype(np.float32)                                    # [chains][V]
        q = np.stack([Q[i][ctx] for i in range(B)], axis=1).astype(np.float32)
        d = orc.sample_drafts(ar, q, seed=123, step=step, flags=orc.FIRST_FROM_TARGET)["tokens"]
        p = np.empty((chains, B + 1, V), np.float32)
        p[:, 0] = ar
        for i in range(1, B + 1):
            p[:, i] = A[d[:, i - 1]]
        o = orc.verify_linear(p, q, d, seed=123, step=step, flags=orc.FIRST_FROM_TARGET)
        for r in range(chains):
            k = o["accept_len"][r]
            toks = o["out_tokens"][r, :k + 1]
            assert (toks >= 0).all()
            committed_counts.append(k + 1)
            prev = ctx[r]
            for t in toks:
                trans[prev, t] += 1
                prev = t
            ctx[r] = prev
    cc = np.array(committed_counts)
    assert cc.min() >= 2 and cc.max() <= B + 1  # 1 <= tokens per forward <= (B+1)/2
    for a in range(V):
        if trans[a].sum() >= 300:
            assert _chisq(trans[a], ref_probs(A[a].astype(np.float32))) > 1e-4, a
