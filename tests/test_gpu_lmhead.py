"""Parity of the LM head + linear verify (psispec_lmhead_verify, through the C ABI) with the
oracle: fp64 logits from the bf16 hidden states and weights (W [H][V], A [H][r], B [r][V]), then the
oracle's linear verify on those fp64 logits.  The call never materialises the logits unless asked
to: the verify outputs of that path are compared with the oracle; with the debug logit buffers the
GPU logits (bf16 MFMA, fp32 accumulation) are compared element by element, and both paths must
give bit-identical outputs (the final draw's recomputed rows equal the first pass's bits)."""
import numpy as np
import pytest
import torch

import oracle
from lossless_draft_verification_spec_amd import PsispecError, psispec_lmhead_verify, workloads
from parity import Tally, compare_linear, gpu_linear_numpy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


class _Ref:
    """Oracle logits of an LM-head input, widened once."""

    def __init__(self, inp):
        pr = inp.preset
        self.b, self.B, self.H, self.V, self.r = pr.batch, pr.B, pr.H, pr.V, pr.r
        self.ha = _bits(inp.h_ar).reshape(self.b * (self.B + 1), self.H)
        self.hd = _bits(inp.h_draft).reshape(self.b * self.B, self.H)
        self.W = oracle.widen_bf16(_bits(inp.W))
        self.A = oracle.widen_bf16(_bits(inp.A)) if self.r else None
        self.Bl = oracle.widen_bf16(_bits(inp.Bl)) if self.r else None

    def rows(self, rq):
        B = self.B
        op = oracle.lmhead_logits_rows(self.ha[rq * (B + 1):(rq + 1) * (B + 1)], self.W)
        oq = oracle.lmhead_logits_rows(self.hd[rq * B:(rq + 1) * B], self.W, self.A, self.Bl, 1.0)
        return op, oq


def _call(inp, d, T, top_p, step, dbg=False, flags=0):
    pr = inp.preset
    dev = lambda x: x.to(DEV)
    kw = {}
    if dbg:
        kw = dict(p_logits_dbg=torch.empty(pr.batch, pr.B + 1, pr.V, device=DEV),
                  q_logits_dbg=torch.empty(pr.batch, pr.B, pr.V, device=DEV))
    out = psispec_lmhead_verify(dev(inp.h_ar), dev(inp.h_draft), dev(inp.W), dev(d),
                                dev(inp.A) if pr.r else None, dev(inp.Bl) if pr.r else None, 1.0,
                                temperature=T, top_p=top_p, seed=inp.seed, step=step, flags=flags,
                                **kw)
    return out, kw


def _run(inp, rows, T=1.0, top_p=1.0, steps=(0,), tally=None, logit_tol=(2e-5, 1e-5), flags=0):
    pr = inp.preset
    B = pr.B
    tally = tally or Tally()
    ref = _Ref(inp)
    orows = {rq: ref.rows(rq) for rq in rows}
    for step in steps:
        d = inp.drafts[step] if step < len(inp.drafts) else inp.drafts[0]
        out_d, dbg = _call(inp, d, T, top_p, step, dbg=True, flags=flags)
        if top_p == 1.0:
            # the production path: no logits in memory; bit-identical to the materialised one
            out_n, _ = _call(inp, d, T, top_p, step, flags=flags)
            gn, gd = gpu_linear_numpy(out_n), gpu_linear_numpy(out_d)
            for k in gn:
                assert np.array_equal(gn[k], gd[k]), k
        g = gpu_linear_numpy(out_d)
        Lp, Lq = dbg["p_logits_dbg"].cpu().numpy(), dbg["q_logits_dbg"].cpu().numpy()
        for rq in rows:
            op, oq = orows[rq]
            atol, rtol = logit_tol
            assert np.allclose(Lp[rq], op, atol=atol, rtol=rtol), np.abs(Lp[rq] - op).max()
            assert np.allclose(Lq[rq], oq, atol=atol, rtol=rtol), np.abs(Lq[rq] - oq).max()
            o = oracle.verify_linear(op[None], oq[None], d.cpu().numpy()[rq:rq + 1], T=T,
                                     top_p=top_p, seed=inp.seed, step=step, request_base=rq,
                                     flags=flags)
            compare_linear(tally, g, o, [rq], B, top_p)
    return tally


@pytest.mark.parametrize("batch,B,H,V,r", [(3, 4, 128, 1000, 16), (1, 1, 64, 296, 0),
                                           (20, 8, 192, 600, 8), (5, 2, 256, 776, 33),
                                           (2, 3, 64, 512, 1), (2, 2, 128, 704, 64),
                                           (11, 12, 320, 2056, 16)])
def test_lmhead_small(batch, B, H, V, r):
    """Ragged row counts (M not a multiple of the 256-row tile), ragged column tiles, LoRA ranks
    0..64 (one to four extra contraction steps), several steps."""
    inp = workloads.make_lmhead("c5", device="cpu", steps=3, batch=batch, B=B, H=H, V=V, r=r)
    t = _run(inp, range(batch), steps=range(3))
    print(t)
    t.check()


def test_lmhead_first_from_target():
    inp = workloads.make_lmhead("c5", device="cpu", steps=2, batch=4, B=5, H=128, V=1000, r=16)
    t = _run(inp, range(4), steps=range(2), flags=1)
    t.check()


def test_lmhead_temperature_top_p():
    inp = workloads.make_lmhead("c5", device="cpu", steps=2, batch=4, B=3, H=128, V=2000, r=16)
    t = _run(inp, range(4), T=0.7, top_p=0.9, steps=range(2))
    t.check()


def test_lmhead_temperature_no_materialise():
    inp = workloads.make_lmhead("c5", device="cpu", steps=2, batch=6, B=4, H=192, V=1536, r=16)
    t = _run(inp, range(6), T=1.6, steps=range(2))
    t.check()


def test_lmhead_top_p_needs_logit_buffers():
    inp = workloads.make_lmhead("c5", device="cpu", steps=1, batch=2, B=2, H=64, V=256, r=0)
    with pytest.raises(PsispecError, match="not implemented"):
        _call(inp, inp.drafts[0], 1.0, 0.9, 0)


def test_lmhead_full_size_sampled_requests():
    """batch 128, B=8, H=4096, V=151936, rank-16 LoRA: the full call on the GPU (with and without
    the logits in memory), sixteen requests over two steps checked against the fp64 oracle."""
    inp = workloads.make_lmhead("c5", device=DEV, steps=2)
    rows = [0, 9, 17, 26, 35, 44, 53, 62, 71, 80, 89, 98, 106, 115, 120, 127]
    t = _run(inp, rows, steps=(0, 1), logit_tol=(5e-5, 1e-5))
    print(t)
    t.check()
