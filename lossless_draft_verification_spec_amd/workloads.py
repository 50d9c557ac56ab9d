"""Seeded synthetic workloads for the Psi-Spec verify step.

This module only draws inputs: logits, drafted tokens and draft trees.  It holds none of the verify
arithmetic (no acceptance test, no residual, no inverse-CDF draw) and imports neither the GPU
library nor the oracle, so both can be fed the very same tensors.  Random numbers come from torch
generators seeded per (workload seed, rotation set, step); draws on a GPU and on the CPU differ, so a
parity check generates once and hands the same tensors to both sides.

The presets follow the five workload descriptions of the verify step (small fp32 case, batch-64 and
batch-256 bf16 blocks with a Zipf boost, large-batch top-p block, prefix tree, fused LM head).  Where
a description leaves a constant open, the reading is stated next to the code.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch


@dataclass(frozen=True)
class LinearPreset:
    name: str
    batch: int
    B: int
    V: int
    dtype: torch.dtype
    T: float = 1.0
    top_p: float = 1.0
    steps: int = 1
    seed: int = 0
    kind: str = "zipf"  # "gauss" (small fp32 case) or "zipf" (bf16 blocks)
    p_std: float = 3.0
    sigmas: tuple = (0.3, 1.0, 2.0)  # draft noise, chosen per request as sigmas[r % len]
    rotations: int = 1
    boost: float = 1.0  # scale of the Zipf boost (2: rows as concentrated as typical LM outputs)


@dataclass(frozen=True)
class TreePreset:
    name: str
    batch: int
    N: int
    depth: int
    k: int
    V: int
    dtype: torch.dtype = torch.float32
    T: float = 1.0
    top_p: float = 1.0
    steps: int = 1
    seed: int = 4
    p_std: float = 3.0
    q_noise: float = 1.0
    peaked: bool = False  # coverage variant: q = p and Zipf-boosted p, so walks go deep
    zipf: bool = False    # Zipf-boosted p as in the linear blocks, q = p + N(0, q_noise^2)
    rotations: int = 1
    boost: float = 1.0    # scale of that Zipf boost


@dataclass(frozen=True)
class LMHeadPreset:
    name: str
    batch: int
    B: int
    H: int
    V: int
    r: int
    T: float = 1.0
    steps: int = 20
    seed: int = 5
    lora_scale: float = 1.0


PRESETS = {
    # 1: batch 1, B=4, V=32, fp32; p ~ N(0, 2^2), q = p rows + N(0, 0.5^2); 10,000 steps
    "c1": LinearPreset("c1", 1, 4, 32, torch.float32, steps=10000, seed=1, kind="gauss", p_std=2.0,
                       sigmas=(0.5,)),
    # 2: batch 64, B=8, V=151936, bf16; N(0, 3^2) + Zipf(1.1) boost on 2% of ids; sigma per request
    "c2": LinearPreset("c2", 64, 8, 151936, torch.bfloat16, steps=200, seed=2, rotations=4),
    # batch-256 block at B=8 (the bandwidth target shape), generated as c2
    "ns": LinearPreset("ns", 256, 8, 151936, torch.bfloat16, steps=200, seed=6, rotations=2),
    # 3: batch 256, B=16, sigma 1.0, T=0.7, top-p 0.95 on p and q
    "c3": LinearPreset("c3", 256, 16, 151936, torch.bfloat16, T=0.7, top_p=0.95, steps=100, seed=3,
                       sigmas=(1.0,), rotations=2),
    # 4: tree, batch 8, depth 8, top-4 candidates, 32 nodes, fp32 rows N(0, 3^2), q = p + N(0, 1)
    "c4": TreePreset("c4", 8, 32, 8, 4, 151936, steps=200, seed=4, rotations=4),
    "c4b": TreePreset("c4b", 8, 32, 8, 4, 151936, steps=20, seed=14, peaked=True),
    # tree with candidates drawn from the draft (recursive rejection), c4's sizes, fp32 rows
    "c4s": TreePreset("c4s", 8, 32, 8, 4, 151936, steps=200, seed=24, rotations=4),
    # 5: fused LM head: batch 128, B=8, H=4096, rank-16 LoRA on the draft rows
    "c5": LMHeadPreset("c5", 128, 8, 4096, 151936, 16),
    # linear-vs-tree batch sweep: one draft/target model for both samplers (bf16, Zipf-boosted
    # N(0, 3^2) target rows, draft = target + N(0, 1)); the batch is set per point of the sweep
    "sweep_linear": LinearPreset("sweep_linear", 1, 8, 151936, torch.bfloat16, steps=50, seed=7,
                                 sigmas=(1.0,)),
    "sweep_tree": TreePreset("sweep_tree", 1, 32, 8, 4, 151936, dtype=torch.bfloat16, steps=50,
                             seed=8, zipf=True),
}


def _gen(device, *keys) -> torch.Generator:
    g = torch.Generator(device=device)
    h = 0x9E3779B97F4A7C15
    for k in keys:
        h = (h ^ (int(k) + 0x632BE59BD9B4E019 + ((h << 6) & (2**64 - 1)) + (h >> 2))) & (2**64 - 1)
    g.manual_seed(h & (2**63 - 1))
    return g


def bf16_bits(t: torch.Tensor) -> torch.Tensor:
    """uint16-compatible view (int16 storage) of a bfloat16 tensor."""
    assert t.dtype == torch.bfloat16
    return t.view(torch.int16)


def zipf_boost(rows: int, V: int, g: torch.Generator, device, frac=0.02, top=10.0, s=1.1):
    """Additive boost: per row, round(frac*V) distinct random ids get random ranks rho = 1..m and
    receive top - s*ln(rho) (>= 1.18 for V = 151936).  Reading of an unspecified 'Zipf(1.1) boost'."""
    m = max(1, int(round(frac * V)))
    keys = torch.rand(rows, V, generator=g, device=device)
    ids = torch.topk(keys, m, dim=1).indices  # random distinct ids in random order
    del keys
    rho = torch.arange(1, m + 1, device=device, dtype=torch.float32)
    vals = (top - s * torch.log(rho)).expand(rows, m)
    boost = torch.zeros(rows, V, device=device, dtype=torch.float32)
    boost.scatter_(1, ids, vals)
    return boost


def nucleus_mask(logits: torch.Tensor, T: float, top_p: float) -> torch.Tensor:
    """Boolean mask of the tie-inclusive nucleus of softmax(logits / T) (draft-side truncation used
    to draw drafted tokens from the truncated draft distribution)."""
    if top_p >= 1.0:
        return torch.ones_like(logits, dtype=torch.bool)
    z = logits.float() / T
    probs = torch.softmax(z.double(), dim=-1)
    sp, idx = torch.sort(probs, dim=-1, descending=True)
    cum = torch.cumsum(sp, dim=-1)
    # first sorted position where the running mass reaches top_p
    cut = torch.searchsorted(cum, torch.full(cum.shape[:-1] + (1,), top_p, dtype=cum.dtype,
                                             device=cum.device))
    cut = cut.clamp(max=logits.shape[-1] - 1)
    thr_logit = torch.gather(logits.float().gather(-1, idx), -1, cut)
    return logits.float() >= thr_logit


def sample_drafts(q: torch.Tensor, T: float, top_p: float, g: torch.Generator) -> torch.Tensor:
    """d_i ~ softmax(q_i / T) restricted to q's nucleus; q[..., B, V] -> int32 [..., B]."""
    shape = q.shape[:-1]
    flat = q.reshape(-1, q.shape[-1])
    out = torch.empty(flat.shape[0], dtype=torch.int64, device=q.device)
    chunk = 1024
    for s in range(0, flat.shape[0], chunk):
        rows = flat[s:s + chunk].float() / T
        if top_p < 1.0:
            mask = nucleus_mask(flat[s:s + chunk], T, top_p)
            rows = rows.masked_fill(~mask, float("-inf"))
        pr = torch.softmax(rows, dim=-1)
        out[s:s + chunk] = torch.multinomial(pr, 1, generator=g).squeeze(-1)
    return out.reshape(shape).to(torch.int32)


@dataclass
class LinearInputs:
    preset: LinearPreset
    p: torch.Tensor  # [batch][B+1][V] float32 or bfloat16
    q: torch.Tensor  # [batch][B][V]
    seed: int        # Philox key for the verify's own uniforms
    drafts: list = field(default_factory=list)  # per step: int32 [batch][B]


def make_linear(preset: LinearPreset | str, device="cpu", rotation: int = 0, steps: int | None = None,
                batch: int | None = None, V: int | None = None, B: int | None = None) -> LinearInputs:
    """Logits of one rotation set plus the drafted tokens of `steps` steps (default: 1)."""
    if isinstance(preset, str):
        preset = PRESETS[preset]
    if batch is not None or V is not None or B is not None:
        preset = replace(preset, batch=batch or preset.batch, V=V or preset.V, B=B or preset.B)
    b, B, V = preset.batch, preset.B, preset.V
    g = _gen(device, preset.seed, rotation, 0xA11CE)
    if preset.kind == "gauss":
        p = torch.randn(b, B + 1, V, generator=g, device=device) * preset.p_std
    else:
        p = torch.randn(b, B + 1, V, generator=g, device=device) * preset.p_std
        p += zipf_boost(b * (B + 1), V, g, device).view(b, B + 1, V) * preset.boost
    sig = torch.tensor([preset.sigmas[r % len(preset.sigmas)] for r in range(b)], device=device,
                       dtype=torch.float32).view(b, 1, 1)
    q = p[:, :B, :] + sig * torch.randn(b, B, V, generator=g, device=device)
    p = p.to(preset.dtype).contiguous()
    q = q.to(preset.dtype).contiguous()
    seed = (preset.seed * 1000003 + rotation) & (2**64 - 1)
    inp = LinearInputs(preset, p, q, seed)
    for s in range(steps if steps is not None else 1):
        inp.drafts.append(draft_step(inp, s))
    return inp


def draft_step(inp: LinearInputs, step: int) -> torch.Tensor:
    g = _gen(inp.p.device, inp.preset.seed, step, 0xD7AF7)
    return sample_drafts(inp.q, inp.preset.T, inp.preset.top_p, g)


@dataclass
class TreeInputs:
    preset: TreePreset
    p: torch.Tensor            # [batch][N+1][V] target logits; row 0 = root, row j+1 = node j
    parent: torch.Tensor       # int32 [batch][N]
    node_tokens: torch.Tensor  # int32 [batch][N]
    seed: int
    q: torch.Tensor | None = None  # [batch][N+1][V] draft logits (sampled candidates only)


def make_tree(preset: TreePreset | str, device="cpu", rotation: int = 0, batch=None, V=None, N=None,
              depth=None, k=None) -> TreeInputs:
    """Prefix trees built best-first by draft path probability (reading of 'pruned by draft
    probability'): each node proposes its top-k draft tokens; the frontier entry with the largest
    product of draft probabilities along its path becomes the next node (ties: lower token id, then
    earlier parent) until N nodes exist; depth never exceeds `depth`.  Node j is scored by row j+1."""
    if isinstance(preset, str):
        preset = PRESETS[preset]
    preset = replace(preset, batch=batch or preset.batch, V=V or preset.V, N=N or preset.N,
                     depth=depth or preset.depth, k=k or preset.k)
    b, N, V, kk = preset.batch, preset.N, preset.V, preset.k
    g = _gen(device, preset.seed, rotation, 0x7EE)
    p = torch.randn(b, N + 1, V, generator=g, device=device) * preset.p_std
    if preset.peaked:
        p += zipf_boost(b * (N + 1), V, g, device).view(b, N + 1, V) * 2.0
        q = p.clone()
    elif preset.zipf:
        p += zipf_boost(b * (N + 1), V, g, device).view(b, N + 1, V) * preset.boost
        q = p + preset.q_noise * torch.randn(b, N + 1, V, generator=g, device=device)
    else:
        q = p + preset.q_noise * torch.randn(b, N + 1, V, generator=g, device=device)
    p = p.to(preset.dtype).contiguous()
    qf = q.float() / preset.T
    # per row: top-k draft candidates and their draft log-probabilities
    logq = torch.log_softmax(qf.double(), dim=-1)
    topv, topi = torch.topk(logq, kk, dim=-1)  # sorted by decreasing draft probability
    topv, topi = topv.cpu(), topi.cpu()
    parent = torch.full((b, N), -1, dtype=torch.int32)
    tokens = torch.zeros((b, N), dtype=torch.int32)
    for r in range(b):
        # frontier entries: (-path_logprob, token, parent_node, parent_row, depth)
        frontier = []
        def push(parent_node, row, base_lp, dep):
            if dep > preset.depth:
                return
            for j in range(kk):
                frontier.append((-(base_lp + float(topv[r, row, j])), int(topi[r, row, j]),
                                 parent_node, dep))
        push(-1, 0, 0.0, 1)
        n = 0
        while n < N and frontier:
            frontier.sort(key=lambda e: (e[0], e[1], e[2]))
            nlp, tok, par, dep = frontier.pop(0)
            parent[r, n] = par
            tokens[r, n] = tok
            push(n, n + 1, -nlp, dep + 1)
            n += 1
        if n < N:
            raise ValueError("tree preset cannot reach N nodes within the depth limit")
    seed = (preset.seed * 1000003 + rotation) & (2**64 - 1)
    return TreeInputs(preset, p, parent.to(device), tokens.to(device), seed)


def make_tree_sampled(preset: TreePreset | str, device="cpu", rotation: int = 0, batch=None, V=None,
                      N=None, branching=(4, 2, 2, 1, 1, 1, 1, 1)) -> TreeInputs:
    """Trees whose candidates are drawn from the draft: the shape is fixed in advance (breadth
    first, branching[d] children for every node at depth d, until N nodes exist), and each child's
    token is drawn independently from its parent's draft row softmax(q / T) restricted to the
    row's nucleus.  The shape must not depend on the drawn tokens for the recursive-rejection rule
    to be lossless, hence the fixed schedule."""
    if isinstance(preset, str):
        preset = PRESETS[preset]
    preset = replace(preset, batch=batch or preset.batch, V=V or preset.V, N=N or preset.N)
    b, N, V = preset.batch, preset.N, preset.V
    g = _gen(device, preset.seed, rotation, 0x5A3)
    p = torch.randn(b, N + 1, V, generator=g, device=device) * preset.p_std
    if preset.zipf or preset.peaked:
        p += zipf_boost(b * (N + 1), V, g, device).view(b, N + 1, V) * preset.boost
    q = p + preset.q_noise * torch.randn(b, N + 1, V, generator=g, device=device)
    p = p.to(preset.dtype).contiguous()
    q = q.to(preset.dtype).contiguous()
    # the fixed shape: parent of every node, breadth first
    parent_list, depth_list = [], []
    frontier = [(-1, 0)]
    while len(parent_list) < N and frontier:
        nxt = []
        for v, d in frontier:
            k = branching[d] if d < len(branching) else 1
            for _ in range(k):
                if len(parent_list) == N or d + 1 > preset.depth:
                    break
                parent_list.append(v)
                depth_list.append(d + 1)
                nxt.append((len(parent_list) - 1, d + 1))
        frontier = nxt
    if len(parent_list) < N:
        raise ValueError("the branching schedule cannot reach N nodes within the depth limit")
    parent = torch.tensor([parent_list] * b, dtype=torch.int32)
    # each child's token from its parent's draft row (row v+1), drawn per node
    par_rows = torch.tensor([v + 1 for v in parent_list], dtype=torch.long, device=device)
    gd = _gen(device, preset.seed, rotation, 0xC4D)
    rows = q[:, par_rows, :]  # [b][N][V]
    tokens = sample_drafts(rows, preset.T, preset.top_p, gd)
    seed = (preset.seed * 1000003 + rotation) & (2**64 - 1)
    return TreeInputs(preset, p, parent.to(device), tokens.to(device), seed, q)


@dataclass
class LMHeadInputs:
    preset: LMHeadPreset
    h_ar: torch.Tensor     # bf16 [batch][B+1][H]
    h_draft: torch.Tensor  # bf16 [batch][B][H]
    W: torch.Tensor        # bf16 [H][V]: the LM-head weight
    A: torch.Tensor        # bf16 [H][r]: LoRA down-projection
    Bl: torch.Tensor       # bf16 [r][V]: LoRA up-projection
    seed: int
    drafts: list = field(default_factory=list)


def make_lmhead(preset: LMHeadPreset | str, device="cpu", rotation: int = 0, steps: int | None = None,
                batch=None, B=None, H=None, V=None, r=None) -> LMHeadInputs:
    """Hidden states ~ N(0,1), W ~ N(0, 0.02^2), LoRA A, B ~ N(0, 0.01^2), all bf16 (independent
    draws for the AR and the draft rows), in the layouts the LM-head call takes: W [H][V],
    A [H][r], B [r][V].  Drafts are drawn from the draft logits computed here with a plain fp32
    torch matmul (input generation only)."""
    if isinstance(preset, str):
        preset = PRESETS[preset]
    preset = replace(preset, batch=batch or preset.batch, B=B or preset.B, H=H or preset.H,
                     V=V or preset.V, r=preset.r if r is None else r)
    b, B, H, V, rr = preset.batch, preset.B, preset.H, preset.V, preset.r
    g = _gen(device, preset.seed, rotation, 0x1AE)
    h_ar = torch.randn(b, B + 1, H, generator=g, device=device).to(torch.bfloat16)
    h_dr = torch.randn(b, B, H, generator=g, device=device).to(torch.bfloat16)
    W = (torch.randn(H, V, generator=g, device=device) * 0.02).to(torch.bfloat16)
    A = (torch.randn(H, max(rr, 1), generator=g, device=device) * 0.01).to(torch.bfloat16)[:, :rr]
    Bl = (torch.randn(max(rr, 1), V, generator=g, device=device) * 0.01).to(torch.bfloat16)[:rr]
    seed = (preset.seed * 1000003 + rotation) & (2**64 - 1)
    inp = LMHeadInputs(preset, h_ar.contiguous(), h_dr.contiguous(), W.contiguous(),
                       A.contiguous(), Bl.contiguous(), seed)
    n = steps if steps is not None else 1
    if n:
        hd = h_dr.float().reshape(b * B, H)
        ql = hd @ W.float()
        if rr:
            ql += preset.lora_scale * ((hd @ A.float()) @ Bl.float())
        ql = ql.view(b, B, V)
        for s in range(n):
            gs = _gen(device, preset.seed, s, 0xD7AF7)
            inp.drafts.append(sample_drafts(ql, preset.T, 1.0, gs))
        del ql
    return inp


def algorithmic_bytes_linear(batch: int, B: int, V: int, elem: int) -> int:
    """Bytes the data-parallel verify must read once: every p row (B+1) and q row (B) of every
    request, plus the drafted tokens and the outputs."""
    return batch * (2 * B + 1) * V * elem + batch * B * 4 + batch * (B + 1) * 4 + batch * (B + 1) * 4


def tree_algorithmic_bytes(batch: int, N: int, V: int, elem: int) -> int:
    return batch * (N + 1) * V * elem + batch * N * 8


def lmhead_flops(batch: int, B: int, H: int, V: int, r: int) -> float:
    M_ar, M_dr = batch * (B + 1), batch * B
    return 2.0 * (M_ar + M_dr) * H * V + 2.0 * M_dr * r * (H + V)

