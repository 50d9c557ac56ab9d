"""Reference distributions for the oracle's pins, written from definitions with library routines
(scipy's softmax, itertools) and no code from the oracle."""
import itertools

import numpy as np
from scipy.special import softmax


def nucleus_set(pi, logits, top_p):
    """Smallest-cardinality set reaching top_p, closed upward under 'logit >=' (ties kept whole)."""
    V = len(pi)
    for n in range(1, V + 1):
        best = None
        for S in itertools.combinations(range(V), n):
            if sum(pi[list(S)]) >= top_p:
                lo = min(logits[list(S)])
                cand = frozenset(x for x in range(V) if logits[x] >= lo)
                if best is None or sum(pi[list(cand)]) < sum(pi[list(best)]):
                    best = cand
        if best is not None:
            return best
    return frozenset(range(V))


def ref_probs(logits, T=1.0, top_p=1.0):
    """softmax(logits / T), then the tie-inclusive nucleus renormalised (small V only)."""
    l = np.asarray(logits, dtype=np.float64)
    finite = np.isfinite(l)
    pi = np.zeros_like(l)
    pi[finite] = softmax(l[finite] / T)
    if top_p >= 1.0:
        return pi
    keep = nucleus_set(pi, np.where(finite, l, -np.inf), top_p)
    out = np.zeros_like(pi)
    idx = sorted(keep)
    out[idx] = pi[idx] / pi[idx].sum()
    return out


def bf16_round(x):
    """float -> bf16 bit patterns, round to nearest even."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_value(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def committed_histogram_check(p_logits, q_logits, accept_len, out_tokens, T=1.0, min_p=1e-4):
    """Repeated-sampling check of losslessness on row-independent targets ([alphalab]
    "為什麼 lossless 不等於答案完全一樣？": fix the settings, sample many times and compare token
    frequencies with confidence bounds).  accept_len[n], out_tokens[n][B+1] from n steps on the same
    logits.  Returns the list of chi-square p-values per position and the mean committed count with
    its closed-form expectation and standard error."""
    from scipy import stats

    Bp1 = p_logits.shape[0]
    B = Bp1 - 1
    pv = [ref_probs(p_logits[j], T) for j in range(Bp1)]
    qv = [ref_probs(q_logits[i], T) for i in range(B)]
    pvals = []
    for j in range(Bp1):
        reached = accept_len >= j
        toks = out_tokens[reached, j]
        n = toks.size
        if n < 200:
            continue
        counts = np.bincount(toks, minlength=len(pv[j])).astype(np.float64)
        exp = n * pv[j]
        big = exp >= 5.0
        obs_b = np.append(counts[big], counts[~big].sum())
        exp_b = np.append(exp[big], exp[~big].sum())
        if exp_b[-1] < 5.0:
            obs_b[-2] += obs_b[-1]
            exp_b[-2] += exp_b[-1]
            obs_b, exp_b = obs_b[:-1], exp_b[:-1]
        pvals.append(stats.chisquare(obs_b, exp_b).pvalue)
    alpha = [np.minimum(pv[i], qv[i]).sum() for i in range(B)]
    reach = np.cumprod([1.0] + alpha)  # P(reach j), j = 0..B
    mean_expected = reach.sum()  # E[committed] = sum_j P(reach j)
    committed = accept_len + 1
    # variance of committed count from its exact law
    probs = np.append(reach[:-1] * (1 - np.array(alpha)), reach[-1])
    vals = np.arange(1, B + 2)
    var = (probs * (vals - mean_expected) ** 2).sum()
    se = np.sqrt(var / committed.size)
    return pvals, committed.mean(), mean_expected, se
