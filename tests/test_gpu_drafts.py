"""Parity of the drafting step of the HIP library (through its C ABI) with the CPU oracle, and an
end-to-end loop on the GPU: draft, verify, commit, over many rounds.

Small and ragged shapes are compared on every drafted token; the full-size blocks (batch 64 x B=8
and batch 256 x B=16 with top-p at V = 151,936) run on the GPU at full size and are compared on
sampled requests."""
import numpy as np
import pytest
import torch
from scipy import stats

from lossless_draft_verification_spec_amd import (PSISPEC_FIRST_FROM_TARGET, ST_NONFINITE,
                                                  psispec_sample_drafts, psispec_verify_linear,
                                                  workloads)
from parity import Tally, compare_drafts, host_logits, oracle_draft_requests

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _rand_rows(batch, B, V, dtype, seed, scale=3.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    p = torch.randn(batch, B + 1, V, generator=g) * scale
    q = p[:, :B] + torch.randn(batch, B, V, generator=g)
    return p.to(dtype).to(DEV), q.to(dtype).to(DEV)


def _compare(q, ar=None, T=1.0, top_p=1.0, seed=99, steps=(0,), flags=0, request_base=0,
             rows=None, tally=None):
    """ar: the tensor handed to the library (None, [batch][V] view or [batch][k][V])."""
    tally = tally or Tally()
    qh = host_logits(q) if q is not None else None
    arh = None
    if ar is not None:
        a = ar if ar.dim() == 3 else ar.unsqueeze(1)
        arh = host_logits(a)
    ref = q if q is not None else ar
    batch = ref.shape[0]
    rows = list(range(batch)) if rows is None else rows
    for step in steps:
        out = psispec_sample_drafts(q, ar_logits=ar, temperature=T, top_p=top_p, seed=seed,
                                    step=step, flags=flags, request_base=request_base)
        torch.cuda.synchronize()
        gt, gs = out["draft_tokens"].cpu().numpy(), out["status"].cpu().numpy()
        V = ref.shape[-1]
        assert ((gt >= 0) & (gt < V)).all()
        o = oracle_draft_requests(arh, qh, rows, float(T), float(top_p), seed, step, flags,
                                  request_base)
        compare_drafts(tally, gt, gs, o, rows, float(top_p))
    return tally


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("batch,B,V", [(1, 4, 32), (5, 3, 1000), (7, 8, 40013), (3, 1, 7),
                                       (2, 64, 300), (4, 16, 4096), (2, 2, 5121)])
def test_drafts_small_and_ragged(dtype, batch, B, V):
    _, q = _rand_rows(batch, B, V, dtype, seed=batch * 100 + B * 7 + V % 89)
    t = _compare(q, steps=range(4))
    print(t)
    t.check()


@pytest.mark.parametrize("T,top_p", [(0.7, 1.0), (1.3, 1.0), (1.0, 0.9), (0.7, 0.95), (1.0, 0.5)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_drafts_temperature_and_top_p(T, top_p, dtype):
    _, q = _rand_rows(6, 5, 5003, dtype, seed=71)
    t = _compare(q, T=T, top_p=top_p, steps=range(3))
    print(t)
    t.check()


@pytest.mark.parametrize("flags", [0, PSISPEC_FIRST_FROM_TARGET])
@pytest.mark.parametrize("T,top_p", [(0.7, 0.95), (1.0, 0.5)])
def test_drafts_fused_row_pass_top_p(T, top_p, flags):
    """bf16 with top-p over at least 256 rows: the row pass and the nucleus share one read."""
    p, q = _rand_rows(40, 8, 4096, torch.bfloat16, seed=17)
    t = _compare(q, ar=p if flags else None, T=T, top_p=top_p, steps=range(3), flags=flags)
    print(t)
    t.check()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_drafts_first_from_target_layouts(dtype):
    batch, B, V = 6, 5, 3000
    p, q = _rand_rows(batch, B, V, dtype, seed=5)
    qn = q.clone()
    qn[:, 0] = float("nan")  # q row 0 is not read in the Uno layout
    F = PSISPEC_FIRST_FROM_TARGET
    # the verify's p tensor: row 0 of each request, stride (B+1) V
    t = _compare(qn, ar=p, flags=F, steps=range(3))
    t.check()
    assert t.status_requests == 0
    full = psispec_sample_drafts(qn, ar_logits=p, seed=3, flags=F)["draft_tokens"]
    # a strided view p[:, 0, :] and a packed copy give the same tokens
    view = psispec_sample_drafts(qn, ar_logits=p[:, 0, :], seed=3, flags=F)["draft_tokens"]
    packed = psispec_sample_drafts(qn, ar_logits=p[:, 0, :].contiguous(), seed=3,
                                   flags=F)["draft_tokens"]
    assert torch.equal(full, view) and torch.equal(full, packed)
    # B = 1 with no q rows at all
    t = _compare(None, ar=p, flags=F, steps=range(2))
    t.check()
    # an odd row stride (not a multiple of 16 bytes) takes the element-wise path
    wide = torch.zeros(batch, V + 3, dtype=dtype, device=DEV)
    wide[:, :V] = p[:, 0]
    t = _compare(qn, ar=wide[:, :V], flags=F, steps=range(2))
    t.check()


@pytest.mark.parametrize("noise", [0.0, 1e-3, 0.05])
def test_drafts_flat_rows(noise):
    """Near-uniform rows over the full vocabulary: the cumulative-weight breakpoints are about S / V
    apart, closer than the bound of the fp32 pass, so many draws are left to the exact fp64 kernels;
    every token must still match the oracle."""
    batch, B, V = 4, 4, 151936
    g = torch.Generator(device="cpu").manual_seed(int(noise * 1e4) + 1)
    q = (torch.randn(batch, B, V, generator=g) * noise).to(DEV)
    t = _compare(q, steps=range(4))
    print(t)
    t.check()
    qb = q.to(torch.bfloat16)
    t = _compare(qb, top_p=0.9, steps=range(2))
    t.check()


def test_drafts_vocab_beyond_bounded_pass():
    """V > 2^21 tokens: more sub-chunks than the bounded select keeps in LDS, so every draw takes the
    exact fp64 kernels (whose select then keeps its sub-chunk masses in the workspace)."""
    _, q = _rand_rows(1, 2, 2100000, torch.bfloat16, seed=21)
    t = _compare(q, steps=range(2))
    t.check()
    t = _compare(q, top_p=0.95, steps=range(1))
    t.check()


def test_drafts_seed_step_request_base_extremes():
    _, q = _rand_rows(4, 4, 777, torch.float32, seed=6)
    t = _compare(q, seed=2**64 - 1, steps=(0, 9, 2**32 - 1), request_base=2**32 - 2)
    t.check()


def test_drafts_status_bits():
    batch, B, V = 4, 3, 500
    _, q = _rand_rows(batch, B, V, torch.float32, seed=10)
    q[1, 2, 7] = float("nan")
    q[2, 0, 9] = float("inf")
    q[3, 1, :] = float("-inf")
    out = psispec_sample_drafts(q, seed=1)
    st = out["status"].cpu().numpy()
    want = np.zeros((batch, B), np.int32)
    want[1, 2] = want[2, 0] = want[3, 1] = ST_NONFINITE
    assert (st & ST_NONFINITE == want).all()
    tok = out["draft_tokens"].cpu().numpy()
    assert ((tok >= 0) & (tok < V)).all()
    t = _compare(q, seed=1)
    assert t.status_requests == 3
    t.check()


def test_drafts_deterministic_and_workspace_independent():
    _, q = _rand_rows(8, 8, 20000, torch.bfloat16, seed=12)
    a = psispec_sample_drafts(q, top_p=0.9, seed=4, step=2)["draft_tokens"].clone()
    ws = torch.full((1 << 26,), 0xFF, dtype=torch.uint8, device=DEV)
    b = psispec_sample_drafts(q, top_p=0.9, seed=4, step=2, workspace=ws)["draft_tokens"]
    assert torch.equal(a, b)


@pytest.mark.parametrize("name,nreq", [("c2", 24), ("c3", 6)])
def test_full_size_drafts(name, nreq):
    inp = workloads.make_linear(name, device=DEV, steps=0)
    pr = inp.preset
    rows = list(range(0, pr.batch, max(1, pr.batch // nreq)))[:nreq]
    qh = host_logits(inp.q)
    tally = Tally()
    for step in range(2):
        out = psispec_sample_drafts(inp.q, temperature=pr.T, top_p=pr.top_p, seed=inp.seed,
                                    step=step)
        torch.cuda.synchronize()
        gt, gs = out["draft_tokens"].cpu().numpy(), out["status"].cpu().numpy()
        assert (gs == 0).all()
        o = oracle_draft_requests(None, qh, rows, pr.T, pr.top_p, inp.seed, step)
        compare_drafts(tally, gt, gs, o, rows, pr.top_p)
    print(name, tally)
    tally.check()


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
    return stats.chisquare(obs_b, exp_b).pvalue


def test_end_to_end_rounds_are_lossless():
    """Draft on the GPU, verify on the GPU, commit, repeat.  The AR is a Markov table over V = 48
    tokens (next-token logits A[last token]); positions 1..B-1 are drafted in parallel from rows that
    depend on the context only.  Committed transitions must follow softmax(A[a]) for every a, and
    every round commits between 2 and B+1 tokens (1 <= tokens per forward <= (B+1)/2)."""
    V, B, chains, rounds = 48, 4, 1024, 30
    rng = np.random.default_rng(17)
    A = torch.tensor(rng.normal(size=(V, V)) * 1.5, dtype=torch.float32, device=DEV)
    Q = A[None] + torch.tensor(rng.normal(size=(B, V, V)), dtype=torch.float32, device=DEV)
    ctx = torch.tensor(rng.integers(0, V, size=chains), dtype=torch.long, device=DEV)
    trans = np.zeros((V, V))
    committed = []
    F = PSISPEC_FIRST_FROM_TARGET
    for step in range(rounds):
        ar = A[ctx].contiguous()
        q = torch.stack([Q[i][ctx] for i in range(B)], dim=1).contiguous()
        d = psispec_sample_drafts(q, ar_logits=ar, seed=31, step=step, flags=F)["draft_tokens"]
        p = torch.empty(chains, B + 1, V, dtype=torch.float32, device=DEV)
        p[:, 0] = ar
        p[:, 1:] = A[d.long()]
        o = psispec_verify_linear(p, q, d, seed=31, step=step, flags=F)
        acc = o["accept_len"].cpu().numpy()
        toks = o["out_tokens"].cpu().numpy()
        c = ctx.cpu().numpy()
        for r in range(chains):
            k = acc[r]
            committed.append(k + 1)
            prev = c[r]
            for t in toks[r, :k + 1]:
                trans[prev, t] += 1
                prev = t
            c[r] = prev
        ctx = torch.tensor(c, dtype=torch.long, device=DEV)
    cc = np.array(committed)
    assert cc.min() >= 2 and cc.max() <= B + 1
    print(f"tokens per forward (committed / 2): {cc.mean() / 2:.3f}")
    Ah = A.cpu().double().numpy()
    pvals = []
    for a in range(V):
        if trans[a].sum() >= 400:
            pr = np.exp(Ah[a] - Ah[a].max())
            pvals.append(_chisq(trans[a], pr / pr.sum()))
    assert len(pvals) >= V // 2
    # one test per context: the smallest p-value of len(pvals) independent tests, Bonferroni
    assert min(pvals) > 1e-4 / len(pvals) * 10, min(pvals)
