"""GPU-vs-oracle comparison rules shared by the parity tests.

* ratios: |gpu - oracle| <= 1e-6 or <= 1e-4 * |oracle|;
* every accept bit, accept_len and every committed token: bit-exact;
* a mismatch is tolerated only when the oracle's margin at the first differing decision is below
  1e-5 (|u - ratio| for an accept test, the normalised CDF gap for the draw, |mass - top_p| at a
  nucleus boundary); tolerated mismatches are counted and must stay below 1e-4 of all decisions.
  Later outputs of a request with a tolerated mismatch are not compared.
* requests whose status is non-zero on either side must have equal status bits (only the
  input-error bits -- non-finite row, bad token, bad parent -- when one of those is set, since the
  other bits then come from arithmetic on invalid data); their other outputs are unspecified.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

ABS, REL, TIE = 1e-6, 1e-4, 1e-5


def host_logits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Tally:
    def __init__(self):
        self.decisions = 0
        self.tolerated = 0
        self.near_ties = 0
        self.requests = 0
        self.status_requests = 0
        self.failures = []

    def check(self):
        assert not self.failures, self.failures[:5]
        assert self.tolerated <= 1e-4 * self.decisions, (self.tolerated, self.decisions)

    def __repr__(self):
        return (f"Tally(requests={self.requests}, decisions={self.decisions}, "
                f"tolerated={self.tolerated}, near_ties={self.near_ties}, "
                f"status_requests={self.status_requests})")


INPUT_ERRORS = oracle.ST_NONFINITE | oracle.ST_BAD_TOKEN | oracle.ST_BAD_PARENT


def _status_equal(sg, so):
    """Input-error bits must agree; when one is set the other bits are unspecified."""
    if (sg | so) & INPUT_ERRORS:
        return (sg & INPUT_ERRORS) == (so & INPUT_ERRORS)
    return sg == so


def _ratio_ok(g, o):
    return np.abs(g - o) <= ABS or np.abs(g - o) <= REL * np.abs(o)


def compare_linear(tally: Tally, g: dict, o: dict, rows, B: int, top_p: float):
    """g: GPU outputs (numpy) for the requests `rows` (indices into g), o: oracle outputs for the
    same requests in the same order."""
    for j, r in enumerate(rows):
        tally.requests += 1
        sg, so = int(g["status"][r]), int(o["status"][j])
        if sg or so:
            tally.status_requests += 1
            if not _status_equal(sg, so):
                tally.failures.append(("status", r, sg, so))
            continue
        ma, ms, mt = o["margin_accept"][j], o["margin_sample"][j], o["margin_topp"][j]
        ndec = B + 1 + ((2 * B + 1) if top_p < 1.0 else 0)
        tally.decisions += ndec
        tally.near_ties += int((ma < TIE).sum()) + int(ms < TIE)
        if top_p < 1.0:
            tally.near_ties += int((mt < TIE).sum())
        topp_tie = top_p < 1.0 and bool((mt < TIE).any())
        gr, orat = g["ratios"][r], o["ratios"][j]
        if not all(_ratio_ok(gr[i], orat[i]) for i in range(B)):
            if topp_tie:
                tally.tolerated += 1
            else:
                tally.failures.append(("ratio", r, gr.tolist(), orat.tolist()))
            continue
        gm, om = int(g["accept_mask"][r]), int(o["accept_mask"][j])
        diff = gm ^ om
        if diff:
            i = (diff & -diff).bit_length() - 1
            if ma[i] < TIE or topp_tie:
                tally.tolerated += 1
            else:
                tally.failures.append(("accept", r, i, float(gr[i]), float(orat[i]), float(ma[i])))
            continue
        k = int(o["accept_len"][j])
        if int(g["accept_len"][r]) != k:
            tally.failures.append(("accept_len", r, int(g["accept_len"][r]), k))
            continue
        gt, ot = g["out_tokens"][r], o["out_tokens"][j]
        if not np.array_equal(gt[:k], ot[:k]) or not np.array_equal(gt[k + 1:], ot[k + 1:]):
            tally.failures.append(("tokens", r, gt.tolist(), ot.tolist()))
            continue
        if gt[k] != ot[k]:
            if ms < TIE or topp_tie:
                tally.tolerated += 1
            else:
                tally.failures.append(("draw", r, int(gt[k]), int(ot[k]), float(ms)))


def compare_tree(tally: Tally, g: dict, o: dict, rows, top_p: float):
    for j, r in enumerate(rows):
        tally.requests += 1
        sg, so = int(g["status"][r]), int(o["status"][j])
        if sg or so:
            tally.status_requests += 1
            if not _status_equal(sg, so):
                tally.failures.append(("status", r, sg, so))
            continue
        ma, ms, mt = o["margin_accept"][j], o["margin_sample"][j], o["margin_topp"][j]
        visited = np.isfinite(ma)
        tally.decisions += int(visited.sum()) + 1 + (len(mt) if top_p < 1.0 else 0)
        tally.near_ties += int((ma[visited] < TIE).sum()) + int(ms < TIE)
        topp_tie = top_p < 1.0 and bool((mt < TIE).any())
        gr, orat = g["node_ratios"][r], o["node_ratios"][j]
        if not all(_ratio_ok(gr[i], orat[i]) for i in range(len(orat))):
            if topp_tie:
                tally.tolerated += 1
            else:
                tally.failures.append(("ratio", r, gr.tolist(), orat.tolist()))
            continue
        dg, do = int(g["accept_len"][r]), int(o["accept_len"][j])
        gn, on = g["accept_nodes"][r], o["accept_nodes"][j]
        if dg != do or not np.array_equal(gn, on):
            # first node where the walks part: tolerated if that accept test was a near tie
            if np.min(ma[visited]) < TIE or topp_tie:
                tally.tolerated += 1
            else:
                tally.failures.append(("walk", r, gn.tolist(), on.tolist()))
            continue
        gt, ot = g["out_tokens"][r], o["out_tokens"][j]
        if not np.array_equal(np.delete(gt, do), np.delete(ot, do)):
            tally.failures.append(("tokens", r, gt.tolist(), ot.tolist()))
            continue
        if gt[do] != ot[do]:
            if ms < TIE or topp_tie:
                tally.tolerated += 1
            else:
                tally.failures.append(("draw", r, int(gt[do]), int(ot[do]), float(ms)))


def gpu_linear_numpy(out: dict) -> dict:
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    res["accept_mask"] = res["accept_mask"].view(np.uint64)
    return res


def oracle_linear_requests(p_host, q_host, drafts_host, rows, T, top_p, seed, step, flags=0,
                           request_base=0):
    """Oracle outputs for the listed requests (each with its own global request id).  The requests
    are independent single-threaded oracle calls; ctypes releases the GIL during each, so they run
    on up to 16 host threads (results in request order)."""
    def one(r):
        return oracle.verify_linear(p_host[r:r + 1], q_host[r:r + 1], drafts_host[r:r + 1], T=T,
                                    top_p=top_p, seed=seed, step=step,
                                    request_base=request_base + r, flags=flags)

    workers = min(16, len(os.sched_getaffinity(0)), max(1, len(rows)))
    if workers > 1:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            outs = list(ex.map(one, rows))
    else:
        outs = [one(r) for r in rows]
    return {k: np.concatenate([o[k] for o in outs]) for k in outs[0]}


def oracle_tree_requests(p_host, parent, tokens, rows, max_depth, T, top_p, seed, step,
                         request_base=0):
    outs = []
    for r in rows:
        o = oracle.verify_tree(p_host[r:r + 1], parent[r:r + 1], tokens[r:r + 1], max_depth, T=T,
                               top_p=top_p, seed=seed, step=step, request_base=request_base + r)
        outs.append(o)
    return {k: np.concatenate([o[k] for o in outs]) for k in outs[0]}


def oracle_tree_sampled_requests(p_host, q_host, parent, tokens, rows, max_depth, T, top_p, seed,
                                 step, request_base=0):
    outs = []
    for r in rows:
        o = oracle.verify_tree_sampled(p_host[r:r + 1], q_host[r:r + 1], parent[r:r + 1],
                                       tokens[r:r + 1], max_depth, T=T, top_p=top_p, seed=seed,
                                       step=step, request_base=request_base + r)
        outs.append(o)
    return {k: np.concatenate([o[k] for o in outs]) for k in outs[0]}


def compare_drafts(tally: Tally, g_tokens, g_status, o: dict, rows, top_p: float):
    """Drafting step: every drafted token is one draw decision (plus one nucleus decision per row
    with top-p).  g_tokens/g_status: GPU [batch][B]; o: oracle outputs of the requests `rows`."""
    for j, r in enumerate(rows):
        tally.requests += 1
        for i in range(g_tokens.shape[1]):
            sg, so = int(g_status[r, i]), int(o["status"][j, i])
            if sg or so:
                tally.status_requests += 1
                if not _status_equal(sg, so):
                    tally.failures.append(("status", r, i, sg, so))
                continue
            ms, mt = o["margin_sample"][j, i], o["margin_topp"][j, i]
            tally.decisions += 2 if top_p < 1.0 else 1
            tally.near_ties += int(ms < TIE) + int(top_p < 1.0 and mt < TIE)
            gt, ot = int(g_tokens[r, i]), int(o["tokens"][j, i])
            if gt != ot:
                if ms < TIE or (top_p < 1.0 and mt < TIE):
                    tally.tolerated += 1
                else:
                    tally.failures.append(("draft", r, i, gt, ot, float(ms)))


def oracle_draft_requests(ar_host, q_host, rows, T, top_p, seed, step, flags=0, request_base=0):
    """Oracle drafting for the listed requests (each with its own global request id); ar_host is
    [batch][k][V] (row 0 read) or None."""
    outs = []
    for r in rows:
        o = oracle.sample_drafts(None if ar_host is None else ar_host[r:r + 1],
                                 None if q_host is None else q_host[r:r + 1], B=1, T=T,
                                 top_p=top_p, seed=seed, step=step, request_base=request_base + r,
                                 flags=flags)
        outs.append(o)
    return {k: np.concatenate([o[k] for o in outs]) for k in outs[0]}
