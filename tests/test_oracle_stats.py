"""Repeated-sampling check of the oracle on the small fp32 workload (batch 1, B=4, V=32,
p ~ N(0, 2^2), q = p + N(0, 0.5^2), T = 1, 10,000 steps): per-position committed-token frequencies
against the target rows (chi-square), and the mean committed count against its closed form
1 + sum_j prod_{i<j} alpha_i with alpha_i = sum_x min(p_i(x), q_i(x))."""
import numpy as np

from lossless_draft_verification_spec_amd import workloads
from refdist import committed_histogram_check


def test_c1_histogram_and_mean_length(orc):
    inp = workloads.make_linear("c1", device="cpu", steps=10000)
    p = inp.p.numpy()
    q = inp.q.numpy()
    n = len(inp.drafts)
    acc = np.zeros(n, np.int32)
    toks = np.zeros((n, inp.preset.B + 1), np.int32)
    for s, d in enumerate(inp.drafts):
        o = orc.verify_linear(p, q, d.numpy(), T=inp.preset.T, seed=inp.seed, step=s)
        acc[s] = o["accept_len"][0]
        toks[s] = o["out_tokens"][0]
    pvals, mean, want, se = committed_histogram_check(p[0], q[0], acc, toks)
    assert len(pvals) >= 3
    assert min(pvals) > 1e-4, pvals
    assert abs(mean - want) < 5 * se, (mean, want, se)
