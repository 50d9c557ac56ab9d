"""Parity of the LM head + linear verify (psispec_lmhead_verify, through the C ABI) with the
oracle: fp64 logits from the bf16 hidden states and weights, then the oracle's linear verify on
those fp64 logits.  The GPU logits (bf16 MFMA, fp32 accumulation) are compared element by element;
the verify outputs follow the same rules as the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_spec_amd import psispec_lmhead_verify, workloads
from parity import Tally, compare_linear, gpu_linear_numpy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _run(inp, rows, T=1.0, top_p=1.0, steps=(0,), tally=None, logit_tol=(2e-5, 1e-5)):
    pr = inp.preset
    b, B, H, V, r = pr.batch, pr.B, pr.H, pr.V, pr.r
    nP = b * (B + 1)
    tally = tally or Tally()
    dev = lambda x: x.to(DEV)
    h_ar, h_dr, w_t = dev(inp.h_ar), dev(inp.h_draft), dev(inp.w_t)
    a_t = dev(inp.a_t) if r else None
    b_t = dev(inp.b_t) if r else None
    logits = torch.empty(b * (2 * B + 1), V, dtype=torch.float32, device=DEV)
    # oracle logits of the sampled requests' rows
    ha, hd = _bits(inp.h_ar).reshape(b * (B + 1), H), _bits(inp.h_draft).reshape(b * B, H)
    wt, at, bt = _bits(inp.w_t), (_bits(inp.a_t) if r else None), (_bits(inp.b_t) if r else None)
    for step in steps:
        d = inp.drafts[step] if step < len(inp.drafts) else inp.drafts[0]
        out = psispec_lmhead_verify(h_ar, h_dr, w_t, dev(d), a_t, b_t, 1.0, temperature=T,
                                    top_p=top_p, seed=inp.seed, step=step, logits=logits)
        g = gpu_linear_numpy(out)
        L = logits.cpu().numpy()
        for rq in rows:
            prow = np.arange(rq * (B + 1), (rq + 1) * (B + 1))
            qrow = nP + np.arange(rq * B, (rq + 1) * B)
            op = oracle.lmhead_logits_rows(ha[prow - 0], wt)
            oq = oracle.lmhead_logits_rows(hd[qrow - nP], wt, at, bt, 1.0)
            atol, rtol = logit_tol
            assert np.allclose(L[prow], op, atol=atol, rtol=rtol), np.abs(L[prow] - op).max()
            assert np.allclose(L[qrow], oq, atol=atol, rtol=rtol), np.abs(L[qrow] - oq).max()
            o = oracle.verify_linear(op[None], oq[None], d.cpu().numpy()[rq:rq + 1], T=T, top_p=top_p,
                                     seed=inp.seed, step=step, request_base=rq)
            compare_linear(tally, g, o, [rq], B, top_p)
    return tally


@pytest.mark.parametrize("batch,B,H,V,r", [(3, 4, 128, 1000, 16), (1, 1, 64, 300, 0),
                                           (20, 8, 192, 600, 8), (5, 2, 256, 777, 33),
                                           (2, 3, 64, 513, 1), (2, 2, 128, 700, 64)])
def test_lmhead_small(batch, B, H, V, r):
    inp = workloads.make_lmhead("c5", device="cpu", steps=3, batch=batch, B=B, H=H, V=V, r=r)
    t = _run(inp, range(batch), steps=range(3))
    print(t)
    t.check()


def test_lmhead_temperature_top_p():
    inp = workloads.make_lmhead("c5", device="cpu", steps=2, batch=4, B=3, H=128, V=2000, r=16)
    t = _run(inp, range(4), T=0.7, top_p=0.9, steps=range(2))
    t.check()


def test_lmhead_full_size_sampled_requests():
    """batch 128, B=8, H=4096, V=151936, rank-16 LoRA: the full call on the GPU, four requests
    checked against the fp64 oracle."""
    inp = workloads.make_lmhead("c5", device=DEV, steps=1)
    t = _run(inp, [0, 45, 90, 127], steps=(0,), logit_tol=(5e-5, 1e-5))
    print(t)
    t.check()
