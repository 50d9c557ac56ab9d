"""Parity of the tree verify with candidates drawn from the draft (recursive rejection) on the GPU
(through the C ABI) with the CPU oracle: small, ragged and full-size trees, temperature and top-p,
draft rows equal to the target rows, too many children, non-finite rows, the caller's bound on
children per node."""
import numpy as np
import pytest
import torch

import oracle

from lossless_draft_verification_spec_amd import (ST_BAD_PARENT, ST_NONFINITE, psispec_verify_tree,
                                                  workloads)
from parity import Tally, compare_tree, host_logits, oracle_tree_sampled_requests

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _compare(tin, T=1.0, top_p=1.0, steps=(0,), rows=None, seed=None, q=None, max_children=0):
    p, q = tin.p, (tin.q if q is None else q)
    ph, qh = host_logits(p), host_logits(q)
    par = tin.parent.cpu().numpy()
    tok = tin.node_tokens.cpu().numpy()
    D = tin.preset.depth
    seed = tin.seed if seed is None else seed
    rows = list(range(p.shape[0])) if rows is None else rows
    tally = Tally()
    for step in steps:
        out = psispec_verify_tree(p, tin.parent, tin.node_tokens, D, temperature=T, top_p=top_p,
                                  seed=seed, step=step, q_logits=q, max_children=max_children)
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in out.items()}
        o = oracle_tree_sampled_requests(ph, qh, par, tok, rows, D, float(T), float(top_p), seed, step)
        compare_tree(tally, g, o, rows, float(top_p))
    return tally


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("batch,N,V,branching", [
    (4, 10, 64, (3, 2, 1)), (3, 32, 5003, (4, 2, 2, 1, 1, 1, 1, 1)), (2, 1, 100, (1,)),
    (5, 40, 999, (8, 2, 1, 1)), (2, 7, 4097, (1, 1, 1, 1, 1, 1, 1)),
    (2, 100, 3001, (8, 3, 2, 1, 1))])
def test_sampled_tree_small(dtype, batch, N, V, branching):
    from dataclasses import replace
    pr = replace(workloads.PRESETS["c4s"], dtype=dtype, depth=8)
    tin = workloads.make_tree_sampled(pr, device=DEV, batch=batch, V=V, N=N, branching=branching)
    t = _compare(tin, steps=range(5))
    print(t)
    t.check()


@pytest.mark.parametrize("N", [63, 64, 65])
@pytest.mark.parametrize("dtype,T,top_p", [(torch.float32, 1.0, 1.0), (torch.bfloat16, 0.7, 0.9)])
def test_sampled_tree_walk_fused_boundary(N, dtype, T, top_p):
    """Trees of up to 64 nodes run their walk inside the draw pass's blocks, larger ones as a
    launch of its own: 63, 64 and 65 nodes on either side of that boundary."""
    from dataclasses import replace
    pr = replace(workloads.PRESETS["c4s"], dtype=dtype, depth=8, T=T, top_p=top_p)
    tin = workloads.make_tree_sampled(pr, device=DEV, batch=3, V=2049, N=N,
                                      branching=(4, 3, 2, 2, 1, 1))
    t = _compare(tin, T=T, top_p=top_p, steps=range(4))
    print(t)
    t.check()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_sampled_tree_max_nodes(dtype):
    """1024 nodes, eight children for every node down to depth 4 (the largest tree and fan-out the
    entry point takes)."""
    from dataclasses import replace
    pr = replace(workloads.PRESETS["c4s"], dtype=dtype, depth=8)
    tin = workloads.make_tree_sampled(pr, device=DEV, batch=2, V=257, N=1024, branching=(8, 8, 8, 8))
    t = _compare(tin, steps=range(3))
    print(t)
    t.check()


@pytest.mark.parametrize("T,top_p", [(0.7, 1.0), (1.0, 0.9), (0.7, 0.95), (1.0, 0.5)])
def test_sampled_tree_temperature_top_p(T, top_p):
    from dataclasses import replace
    pr = replace(workloads.PRESETS["c4s"], dtype=torch.bfloat16, T=T, top_p=top_p)
    tin = workloads.make_tree_sampled(pr, device=DEV, batch=4, V=3001, N=24)
    t = _compare(tin, T=T, top_p=top_p, steps=range(4))
    print(t)
    t.check()


def test_equal_draft_accepts_first_children():
    tin = workloads.make_tree_sampled("c4s", device=DEV, batch=3, V=2000, N=20)
    out = psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, 8, seed=1, q_logits=tin.p)
    par = tin.parent[0].cpu().numpy()
    first_path = []
    v = -1
    while True:
        kids = [c for c in range(len(par)) if par[c] == v]
        if not kids:
            break
        first_path.append(kids[0])
        v = kids[0]
    acc = out["accept_len"].cpu().numpy()
    nodes = out["accept_nodes"].cpu().numpy()
    assert (acc == len(first_path)).all()
    assert (nodes[:, :len(first_path)] == np.array(first_path)).all()
    t = _compare(tin, q=tin.p)
    t.check()


def test_too_many_children_and_nonfinite_rows():
    tin = workloads.make_tree_sampled("c4s", device=DEV, batch=3, V=500, N=12,
                                      branching=(9, 1, 1))
    out = psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, 8, seed=2, q_logits=tin.q)
    assert (out["status"].cpu().numpy() & ST_BAD_PARENT).all()
    tin = workloads.make_tree_sampled("c4s", device=DEV, batch=3, V=500, N=12)
    q = tin.q.clone()
    q[1, 0, 7] = float("nan")
    out = psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, 8, seed=2, q_logits=q)
    st = out["status"].cpu().numpy()
    assert st[1] & ST_NONFINITE and not (st[0] & ST_NONFINITE) and not (st[2] & ST_NONFINITE)
    t = _compare(tin, q=q)
    assert t.status_requests >= 1
    t.check()


def test_full_size_sampled_tree():
    tin = workloads.make_tree_sampled("c4s", device=DEV)
    t = _compare(tin, steps=range(2), rows=[0, 3, 7])
    print(t)
    t.check()


def _ratio_band_tokens(tin, picks):
    """fp32 rows in which chosen tokens of a node's draft row have p'(x) / q'(x) equal to 1 up to
    the logits' fp32 rounding (their q logit set from the exact normalisers, a few fixed-point
    rounds): the tokens where the sign of p' - q' is closest to undecided.  picks: (request, node
    row, token indices)."""
    q = tin.q.detach().cpu().double().clone()
    p = tin.p.detach().cpu().double()
    for r, row, xs in picks:
        lp, lq = p[r, row], q[r, row]
        xs = torch.as_tensor(xs)
        for _ in range(4):
            Ep = torch.exp(lp - lp.max()).sum()
            Eq = torch.exp(lq - lq.max()).sum()
            lq[xs] = lp[xs] - lp.max() + lq.max() - torch.log(Ep / Eq)
        q[r, row] = lq
    return q.to(torch.float32).to(DEV)


def test_ratio_band_tokens():
    """Tokens whose ratio p'/q' sits at 1 within the logits' rounding: a few per chunk (the level-0
    split keeps them and the resolve settles them in index order) and many in one chunk (that chunk
    is recomputed in full, the others keep the split)."""
    tin = workloads.make_tree_sampled("c4s", device=DEV, batch=3, V=40000, N=20)
    p = tin.p.detach().cpu()
    picks = []
    for r in range(3):
        low = torch.argsort(p[r, 0])[:400].sort().values  # low target logits: q stays below its max
        few = [int(x) for x in low[::57][:6]]
        chunk0 = [int(x) for x in low if x < 4096][:14]  # more than a chunk keeps
        picks.append((r, 0, few + chunk0 if r == 1 else few))
        low1 = torch.argsort(p[r, 1])[:50]
        picks.append((r, 1, [int(x) for x in low1[:3]]))
    q = _ratio_band_tokens(tin, picks)
    t = _compare(tin, steps=range(3), q=q)
    print(t)
    t.check()


def test_chain_passes_over_several_grid_rounds():
    """A call whose chain passes take more than one round of their fixed grids: 14,336 node rows x
    38 chunks = 544,768 items (one round covers about 2048 x 256 items at level 1 and 509 x 256 from
    level 2 on), nodes with 3 to 8 children (levels 1-7 have work), and in a few nodes' draft rows
    more in-between tokens of the level-0 split than a chunk keeps, all in the row's last chunk, so
    that level 1 recomputes chunks that only its second round reaches.  Sampled requests against the
    oracle."""
    from dataclasses import replace
    pr = replace(workloads.PRESETS["c4s"], dtype=torch.float32, depth=8)
    tin = workloads.make_tree_sampled(pr, device=DEV, batch=56, V=151936, N=255,
                                      branching=(8, 4, 3, 3))
    par = tin.parent.cpu().numpy()
    V = tin.p.shape[2]
    last0 = (V - 1) // 4096 * 4096  # first token of the last 4096-token chunk
    picks = []
    for r in (2, 30, 55):
        kids = np.bincount(par[r] + 1, minlength=par.shape[1] + 1)
        rows = [int(v) for v in np.nonzero(kids >= 2)[0][:3]]  # node rows with two or more children
        for row in rows:
            lp = tin.p[r, row, last0:].cpu()
            picks.append((r, row, [last0 + int(x) for x in torch.argsort(lp)[:12]]))
    q = tin.q
    for r, row, xs in picks:
        lp = tin.p[r, row].detach().cpu().double()
        lq = q[r, row].detach().cpu().double().clone()
        xs = torch.as_tensor(xs)
        for _ in range(4):
            Ep = torch.exp(lp - lp.max()).sum()
            Eq = torch.exp(lq - lq.max()).sum()
            lq[xs] = lp[xs] - lp.max() + lq.max() - torch.log(Ep / Eq)
        q[r, row] = lq.to(torch.float32).to(DEV)
    rows = [2, 30, 55]
    tally = Tally()
    for step in range(2):
        out = psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, 8, seed=tin.seed, step=step,
                                  q_logits=q)
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in out.items()}
        outs = []
        for r in rows:
            outs.append(oracle.verify_tree_sampled(
                host_logits(tin.p[r:r + 1]), host_logits(q[r:r + 1]), par[r:r + 1],
                tin.node_tokens[r:r + 1].cpu().numpy(), 8, T=1.0, top_p=1.0, seed=tin.seed,
                step=step, request_base=r))
        o = {k: np.concatenate([x[k] for x in outs]) for k in outs[0]}
        compare_tree(tally, g, o, rows, 1.0)
    print(tally)
    tally.check()


def _verify(tin, **kw):
    out = psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, tin.preset.depth, seed=tin.seed,
                              q_logits=tin.q, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("N,branching,bounds", [
    (30, (4, 2, 2, 1, 1, 1, 1, 1), (4, 5, 8)), (7, (1,) * 7, (1, 2)), (40, (8, 2, 1, 1), (8,)),
    (20, (2, 3, 1, 1), (3, 6))])
def test_max_children_bound_same_outputs(dtype, N, branching, bounds):
    """A bound on children per node at or above the tree's largest fan-out gives the outputs of the
    call without it, bit for bit (the passes it skips have no node to work on), and they agree with
    the oracle."""
    from dataclasses import replace
    pr = replace(workloads.PRESETS["c4s"], dtype=dtype, depth=8)
    tin = workloads.make_tree_sampled(pr, device=DEV, batch=4, V=3001, N=N, branching=branching)
    for step in (0, 1):
        base = _verify(tin, step=step)
        for k in bounds:
            got = _verify(tin, step=step, max_children=k)
            for key in base:
                np.testing.assert_array_equal(got[key], base[key], err_msg=f"{key} bound {k}")
    t = _compare(tin, steps=range(2), max_children=bounds[0])
    print(t)
    t.check()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_max_children_bound_below_fanout(dtype):
    """Requests holding a node with more children than the bound are reported with ST_BAD_PARENT;
    the other requests of the same call keep the outputs of the call without the bound."""
    from dataclasses import replace
    pr = replace(workloads.PRESETS["c4s"], dtype=dtype, depth=8)
    wide = workloads.make_tree_sampled(pr, device=DEV, batch=2, V=2000, N=24,
                                       branching=(4, 2, 2, 1, 1))
    narrow = workloads.make_tree_sampled(pr, device=DEV, batch=2, V=2000, N=24, rotation=1,
                                         branching=(2, 2, 2, 1, 1))
    cat = lambda a, b: torch.cat([a, b]).contiguous()
    mixed = replace(wide, p=cat(wide.p, narrow.p), q=cat(wide.q, narrow.q),
                    parent=cat(wide.parent, narrow.parent),
                    node_tokens=cat(wide.node_tokens, narrow.node_tokens))
    base = _verify(mixed, top_p=0.9)
    for k in (2, 3):
        got = _verify(mixed, top_p=0.9, max_children=k)
        assert (got["status"][:2] & ST_BAD_PARENT).all()
        assert not (got["status"][2:] & ST_BAD_PARENT).any()
        for key in base:
            np.testing.assert_array_equal(got[key][2:], base[key][2:], err_msg=f"{key} bound {k}")
    got = _verify(mixed, top_p=0.9, max_children=1)
    assert (got["status"] & ST_BAD_PARENT).all()
    t = _compare(mixed, top_p=0.9, steps=range(2))
    t.check()
