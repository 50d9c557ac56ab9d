"""The linear verify's no-allocation entry point (psispec_verify_linear_noalloc, through the C ABI)
against the entry point with a caller workspace: bit-identical outputs on two calls in a row, the
second smaller, and a clear error for sizes beyond its fixed scratch."""
import numpy as np
import pytest
import torch

from lossless_draft_verification_spec_amd import (PsispecError, psispec_verify_linear,
                                                  psispec_verify_linear_noalloc, workloads)
from parity import gpu_linear_numpy

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(batch, B, V, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    p = torch.randn(batch, B + 1, V, generator=g) * 3.0
    q = p[:, :B] + torch.randn(batch, B, V, generator=g)
    p, q = p.to(dtype), q.to(dtype)
    d = workloads.sample_drafts(q, 1.0, 1.0, g)
    return p.to(DEV), q.to(DEV), d.to(DEV)


def _out(batch, B):
    return dict(accept_len=torch.full((batch,), -7, dtype=torch.int32, device=DEV),
                out_tokens=torch.full((batch, B + 1), -7, dtype=torch.int32, device=DEV),
                ratios=torch.full((batch, B), -7.0, dtype=torch.float32, device=DEV),
                accept_mask=torch.zeros(batch, dtype=torch.int64, device=DEV),
                status=torch.full((batch,), -7, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("first,second", [((256, 8, 151936, torch.bfloat16, 1.0),
                                           (5, 3, 1000, torch.float32, 0.9)),
                                          ((64, 16, 20000, torch.bfloat16, 0.95),
                                           (1, 1, 7, torch.bfloat16, 1.0))])
def test_noalloc_matches_workspace_entry_point(first, second):
    for k, (batch, B, V, dtype, top_p) in enumerate((first, second)):
        p, q, d = _inputs(batch, B, V, dtype, seed=31 + k)
        ref = gpu_linear_numpy(psispec_verify_linear(p, q, d, top_p=top_p, seed=9, step=k,
                                                     request_base=3))
        got = psispec_verify_linear_noalloc(p, q, d, _out(batch, B), top_p=top_p, seed=9, step=k,
                                            request_base=3)
        torch.cuda.synchronize()
        got = gpu_linear_numpy(got)
        for key in ref:
            assert np.array_equal(ref[key], got[key]), (key, batch, B, V)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    batch, B = 600, 8
    # a [600][9][151936] call needs more than 64 MiB of scratch (never launched)
    p = torch.empty(batch, B + 1, 151936, dtype=torch.bfloat16, device=DEV)
    q = torch.empty(batch, B, 151936, dtype=torch.bfloat16, device=DEV)
    d = torch.zeros(batch, B, dtype=torch.int32, device=DEV)
    with pytest.raises(PsispecError, match="scratch"):
        psispec_verify_linear_noalloc(p, q, d, _out(batch, B))
