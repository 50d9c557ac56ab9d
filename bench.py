#!/usr/bin/env python3
"""Benchmark of the Psi-Spec linear verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one psispec_verify_linear call over one batch of synthetic logits: the HBM pass over
every p and q row, the nucleus pass when top-p is on, the accept test and first-rejection scan, and
the fp64 final draw.  The timed workload is the batch-64, B=8, V=151,936 bf16 block (Zipf-boosted
N(0, 3^2) target logits, draft noise sigma in {0.3, 1, 2} per request, T = 1); rotation sets that
together exceed the 256 MB last-level cache are cycled so every step reads its rows from HBM, and
each step has its own drafted tokens and Philox step.  Inputs are resident in HBM before timing.

One JSON line is printed: verified rows/s (batch*B per step) as `value`, committed tokens/s, the
roofline of the dominant kernel (the HBM pass, timed with HIP events on the library's stream), the
oracle timed on the host cores as `cpu_baseline`, the batch-256 B=8 shape as `target_shape`, the
LM head + verify (batch 128, B=8, H=4096, rank-16 LoRA) with its MFMA roofline as `lmhead`, and the
32-node tree verify as `tree`, the drafting step (batch 64, B=8, Uno layout) as `drafts`, and the
KV commit after tree verifies (batch 256, 114,688-byte rows) as `kv_commit`.
`--workload c3|c4|c5|drafts|kv` prints the top-p, tree, LM-head, drafting or KV-commit line alone;
`--workload sweep` prints the linear-vs-tree batch sweep (batch 1..256).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, datasheet
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2",
                    choices=["c2", "ns", "c3", "c4", "c4s", "c5", "drafts", "sweep", "kv"])
    ap.add_argument("--sweep-batches", default="1,2,4,8,16,32,64,128,256",
                    help="batch sizes of the linear-vs-tree sweep")
    ap.add_argument("--sweep-steps", type=int, default=40)
    ap.add_argument("--sweep-noise", type=float, default=1.0,
                    help="draft noise sigma of the sweep (draft = target + N(0, sigma^2))")
    ap.add_argument("--sweep-boost", type=float, default=1.0,
                    help="Zipf boost scale of the sweep's target rows (2: concentrated rows)")
    ap.add_argument("--no-lmhead", action="store_true", help="skip the fused LM-head measurement")
    ap.add_argument("--lmhead-steps", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-target", action="store_true", help="skip the batch-256 target shape")
    ap.add_argument("--no-tree", action="store_true", help="skip the tree verify measurement")
    ap.add_argument("--tree-steps", type=int, default=100)
    ap.add_argument("--no-drafts", action="store_true", help="skip the drafting-step measurement")
    ap.add_argument("--no-kv", action="store_true", help="skip the KV-commit measurement")
    ap.add_argument("--kv-steps", type=int, default=50)
    ap.add_argument("--draft-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter scaling)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def run_workload(name, steps, warmup, torch, pkg, workloads):
    """Time `steps` verify calls; returns a dict of measurements."""
    preset = workloads.PRESETS[name]
    R = preset.rotations
    per_rot = (steps + warmup + R - 1) // R + 1
    t0 = time.time()
    sets = [workloads.make_linear(preset, device="cuda", rotation=i, steps=per_rot) for i in range(R)]
    torch.cuda.synchronize()
    log(f"{name}: generated {R} rotation sets in {time.time() - t0:.1f}s")
    b, B, V = preset.batch, preset.B, preset.V
    dev = sets[0].p.device
    ws = torch.empty(pkg.linear_workspace_bytes(b, B, V, pkg.PSISPEC_BF16), dtype=torch.uint8,
                     device=dev)
    n_total = steps + warmup
    acc_all = torch.zeros(n_total, b, dtype=torch.int32, device=dev)
    outs = [dict(accept_len=acc_all[s],
                 out_tokens=torch.empty(b, B + 1, dtype=torch.int32, device=dev),
                 ratios=torch.empty(b, B, dtype=torch.float32, device=dev),
                 accept_mask=torch.empty(b, dtype=torch.int64, device=dev),
                 status=torch.empty(b, dtype=torch.int32, device=dev)) for s in range(min(n_total, 8))]

    def step(s, out):
        inp = sets[s % R]
        d = inp.drafts[s // R]
        o = dict(outs[s % len(outs)])
        o["accept_len"] = acc_all[s]
        pkg.psispec_verify_linear(inp.p, inp.q, d, temperature=preset.T, top_p=preset.top_p,
                                  seed=inp.seed, step=s, workspace=ws, out=o)

    for s in range(warmup):
        step(s, None)
    torch.cuda.synchronize()
    # phase A: the timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for s in range(warmup, warmup + steps):
        step(s, None)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = ev0.elapsed_time(ev1)
    committed = int((acc_all[warmup:warmup + steps].to(torch.int64) + 1).sum().item())
    # phase B: same steps again with HIP events around every library kernel
    pkg.timing_enable(True)
    for s in range(warmup, warmup + steps):
        step(s, None)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    torch.cuda.synchronize()
    elem = 2 if preset.dtype == torch.bfloat16 else 4
    alg = workloads.algorithmic_bytes_linear(b, B, V, elem)
    row_bytes = b * (2 * B + 1) * V * elem
    res = dict(name=name, preset=preset, ms_total=ms, wall_s=wall, steps=steps,
               ms_per_step=ms / steps, rows_per_s=steps * b * B / (ms / 1e3),
               committed_per_s=committed / (ms / 1e3), alg_bytes=alg, row_bytes=row_bytes,
               kernels={k: dict(avg_us=1e3 * v[0] / max(1, v[1]), launches=v[1])
                        for k, v in kern.items()},
               mean_committed=committed / (steps * b))
    res["hbm_gbs_step"] = alg / (res["ms_per_step"] / 1e3) / 1e9
    # the pass that reads every p and q row: the row pass, or the row pass fused with the nucleus
    res["row_kernel"] = "rowstats" if "rowstats" in res["kernels"] else "rowstats_topp"
    rs = res["kernels"].get(res["row_kernel"])
    if rs:
        res["rowstats_gbs"] = row_bytes / (rs["avg_us"] / 1e6) / 1e9
    host = dict(p=sets[0].p, q=sets[0].q, d=sets[0].drafts[0], seed=sets[0].seed)
    del sets
    torch.cuda.empty_cache()
    return res, host


def run_tree(steps, warmup, torch, pkg, workloads, name="c4"):
    """Time psispec_verify_tree on the 8-request, 32-node, V=151936 fp32 tree workload (rotation
    sets exceeding the last-level cache); HBM roofline of the row pass over the N+1 node rows (and
    the N+1 draft rows for `c4s`, whose candidates are drawn from the draft and verified by
    recursive rejection)."""
    preset = workloads.PRESETS[name]
    sampled = name == "c4s"
    R = preset.rotations
    t0 = time.time()
    make = workloads.make_tree_sampled if sampled else workloads.make_tree
    sets = [make(preset, device="cuda", rotation=i) for i in range(R)]
    torch.cuda.synchronize()
    log(f"{name}: generated {R} rotation sets in {time.time() - t0:.1f}s")
    b, N, V = preset.batch, preset.N, preset.V
    elem = 2 if preset.dtype == torch.bfloat16 else 4
    dt = pkg.PSISPEC_BF16 if elem == 2 else pkg.PSISPEC_F32
    ws = torch.empty(pkg.tree_workspace_bytes(b, N, V, dt), dtype=torch.uint8, device="cuda")
    acc = torch.zeros(b, dtype=torch.int64, device="cuda")

    def step(s):
        inp = sets[s % R]
        return pkg.psispec_verify_tree(inp.p, inp.parent, inp.node_tokens, preset.depth,
                                       temperature=preset.T, top_p=preset.top_p, seed=inp.seed,
                                       step=s, workspace=ws, q_logits=inp.q if sampled else None)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(warmup, warmup + steps):
        o = step(s)
        acc += o["accept_len"].to(torch.int64) + 1
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    committed = int(acc.sum().item())
    pkg.timing_enable(True)
    for s in range(warmup, warmup + steps):
        step(s)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    row_bytes = b * (N + 1) * V * elem * (2 if sampled else 1)
    rs = kern.get("rowstats", (0.0, 1))
    rs_us = 1e3 * rs[0] / max(1, rs[1])
    del sets
    torch.cuda.empty_cache()
    rule = "candidates drawn from the draft (recursive rejection)" if sampled else \
        "top-4 candidates"
    return dict(workload=f"{name}: tree verify batch={b} N={N} nodes depth<={preset.depth} V={V} "
                         f"{'bf16' if elem == 2 else 'fp32'} logits, T={preset.T}, {rule}",
                ms_per_step=round(ms / steps, 4),
                nodes_per_s=round(steps * b * N / (ms / 1e3), 1),
                committed_tokens_per_s=round(committed / (ms / 1e3), 1),
                mean_committed_per_request=round(committed / (steps * b), 4),
                kernels_avg_us={k: round(1e3 * v[0] / max(1, v[1]), 2) for k, v in kern.items()},
                roofline={"bound": "hbm", "kernel": "k_rowstats",
                          "achieved": round(row_bytes / (rs_us / 1e6) / 1e9, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(row_bytes / (rs_us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": row_bytes, "avg_launch_us": round(rs_us, 2)})


def run_drafts(steps, warmup, torch, pkg, workloads, name="c2"):
    """Time psispec_sample_drafts on the batch-64, B=8, V=151936 bf16 block in the Uno layout: d_0
    from the AR row (row 0 of the verify's p tensor, read in place), d_1..d_7 from q rows 1..7.
    Rotation sets exceed the last-level cache.  HBM roofline of the bounded fp32 pass, which reads
    the B sampled rows of every request once; the exact fp64 kernels that settle the remaining
    draws are timed beside it (draw_pass, draw_select)."""
    preset = workloads.PRESETS[name]
    R = preset.rotations
    t0 = time.time()
    sets = [workloads.make_linear(preset, device="cuda", rotation=i, steps=0) for i in range(R)]
    torch.cuda.synchronize()
    log(f"drafts ({name}): generated {R} rotation sets in {time.time() - t0:.1f}s")
    b, B, V = preset.batch, preset.B, preset.V
    elem = 2 if preset.dtype == torch.bfloat16 else 4
    dt = pkg.PSISPEC_BF16 if elem == 2 else pkg.PSISPEC_F32
    ws = torch.empty(pkg.drafts_workspace_bytes(b, B, V, dt), dtype=torch.uint8, device="cuda")
    out = dict(draft_tokens=torch.empty(b, B, dtype=torch.int32, device="cuda"),
               status=torch.empty(b, B, dtype=torch.int32, device="cuda"))
    F = pkg.PSISPEC_FIRST_FROM_TARGET

    def step(s):
        inp = sets[s % R]
        pkg.psispec_sample_drafts(inp.q, ar_logits=inp.p, temperature=preset.T, top_p=preset.top_p,
                                  seed=inp.seed, step=s, flags=F, workspace=ws, out=out)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(warmup, warmup + steps):
        step(s)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    pkg.timing_enable(True)
    for s in range(warmup, warmup + steps):
        step(s)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    row_bytes = b * B * V * elem  # every sampled row read once
    k_us = {k: 1e3 * v[0] / max(1, v[1]) for k, v in kern.items()}
    bd_us = k_us.get("draft_bounds", 0.0)
    del sets
    torch.cuda.empty_cache()
    gbs = row_bytes / (bd_us / 1e6) / 1e9 if bd_us > 0 else 0.0
    return dict(workload=f"drafts ({name}): Uno-layout drafting batch={b} B={B} V={V} "
                         f"{'bf16' if elem == 2 else 'fp32'} logits, T={preset.T}, "
                         f"top_p={preset.top_p}",
                ms_per_step=round(ms / steps, 4),
                drafted_tokens_per_s=round(steps * b * B / (ms / 1e3), 1),
                hbm_gbs_step=round(row_bytes / (ms / steps / 1e3) / 1e9, 1),
                kernels_avg_us={k: round(v, 2) for k, v in k_us.items()},
                roofline={"bound": "hbm", "kernel": "k_draft_bounds", "achieved": round(gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "traffic": read_traffic("draft_bounds", name),
                          "bytes_per_launch": row_bytes, "avg_launch_us": round(bd_us, 2)})


def _time_calls(torch, pkg, call, steps, warmup):
    """Mean device time per call (torch events over `steps` calls after `warmup`), the summed
    outputs of the timed calls, and the library's per-kernel mean times (a second pass)."""
    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    outs = []
    ev0.record()
    for s in range(warmup, warmup + steps):
        outs.append(call(s))
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    pkg.timing_enable(True)
    for s in range(warmup, warmup + steps):
        call(s)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    return ms / steps, outs, {k: 1e3 * v[0] / max(1, v[1]) for k, v in kern.items()}


def run_sweep(batches, steps, torch, pkg, workloads, noise=1.0, boost=1.0):
    """Linear vs tree verify over batch sizes at fixed B=8 (linear) and N=32, depth <= 8, top-4
    (tree), V=151936 bf16, one draft/target model for both (N(0, 3^2) target rows plus `boost` times
    the Zipf boost, draft = target + N(0, noise^2)).  Each point cycles rotation sets totalling >= 600 MB so every
    call reads its rows from HBM.  Per point: device time per call, committed tokens per call and per
    second, rows read per call and the row pass's share of HBM peak."""
    from dataclasses import replace
    pl = replace(workloads.PRESETS["sweep_linear"], sigmas=(noise,), boost=boost)
    pt = replace(workloads.PRESETS["sweep_tree"], q_noise=noise, boost=boost)
    V, B, N = pl.V, pl.B, pt.N
    points = []
    for b in batches:
        lin_bytes, tree_bytes = b * (2 * B + 1) * V * 2, b * (N + 1) * V * 2
        R = max(2, min(64, -(-600_000_000 // lin_bytes)))
        sets = [workloads.make_linear(pl, device="cuda", rotation=i, batch=b,
                                      steps=(steps + 3) // R + 2) for i in range(R)]
        ws = torch.empty(pkg.linear_workspace_bytes(b, B, V, pkg.PSISPEC_BF16), dtype=torch.uint8,
                         device="cuda")

        def lin(s):
            inp = sets[s % R]
            return pkg.psispec_verify_linear(inp.p, inp.q, inp.drafts[s // R], seed=inp.seed,
                                             step=s, workspace=ws)["accept_len"]

        ms_l, acc_l, k_l = _time_calls(torch, pkg, lin, steps, 3)
        com_l = float(sum((a.to(torch.int64) + 1).sum().item() for a in acc_l)) / steps
        del sets, ws
        Rt = max(2, min(64, -(-600_000_000 // tree_bytes)))
        tsets = [workloads.make_tree(pt, device="cuda", rotation=i, batch=b) for i in range(Rt)]
        wst = torch.empty(pkg.tree_workspace_bytes(b, N, V, pkg.PSISPEC_BF16), dtype=torch.uint8,
                          device="cuda")

        def tree(s):
            inp = tsets[s % Rt]
            return pkg.psispec_verify_tree(inp.p, inp.parent, inp.node_tokens, pt.depth,
                                           seed=inp.seed, step=s, workspace=wst)["accept_len"]

        ms_t, acc_t, k_t = _time_calls(torch, pkg, tree, steps, 3)
        com_t = float(sum((a.to(torch.int64) + 1).sum().item() for a in acc_t)) / steps
        del tsets, wst
        torch.cuda.empty_cache()

        def leg(ms, com, rows, nbytes, k):
            rs = k.get("rowstats", 0.0)
            return dict(us_per_call=round(1e3 * ms, 2), committed_per_call=round(com, 3),
                        committed_tokens_per_s=round(com / (ms / 1e3), 1), rows_per_call=rows,
                        rowstats_us=round(rs, 2),
                        rowstats_frac_of_hbm_peak=round(nbytes / (rs / 1e6) / 1e9 / HBM_PEAK_GBS, 4)
                        if rs > 0 else None,
                        kernels_avg_us={kk: round(v, 2) for kk, v in k.items()})

        pt_ = dict(batch=b, linear=leg(ms_l, com_l, b * (2 * B + 1), lin_bytes, k_l),
                   tree=leg(ms_t, com_t, b * (N + 1), tree_bytes, k_t))
        log(f"sweep batch {b}: linear {pt_['linear']['us_per_call']} us "
            f"{pt_['linear']['committed_tokens_per_s']:.0f} tok/s; tree {pt_['tree']['us_per_call']} us "
            f"{pt_['tree']['committed_tokens_per_s']:.0f} tok/s")
        points.append(pt_)
    return dict(workload=f"linear (B={B}) vs tree (N={N}, depth<={pt.depth}, top-{pt.k}) verify, "
                         f"V={V} bf16, N(0,3^2) target rows + {boost} x Zipf boost, draft = "
                         f"target + N(0,{noise}^2), T=1",
                steps_per_point=steps, points=points)


KV_ROW_BYTES = 28 * 2 * 8 * 128 * 2  # one position: 28 layers x (K, V) x 8 KV heads x 128 dims, bf16


def run_kv(steps, warmup, torch, pkg, workloads):
    """Time psispec_kv_commit after tree verifies: batch 256 lines of 160 positions of 114,688-byte
    rows (4.7 GB), 32-position blocks; the kept paths are the accepted nodes of tree verifies of the
    concentrated sweep workload (N=32, depth <= 8, top-4, V=151936 bf16), one set per step, and each
    step has its own line lengths.  HBM roofline of the copy kernel over the bytes it must move (each
    moved row read once and written once)."""
    from dataclasses import replace
    b, Lmax, blk = 256, 160, 32
    pt = replace(workloads.PRESETS["sweep_tree"], boost=2.0)
    tin = workloads.make_tree(pt, device="cuda", batch=b)
    n_all, keep_all = [], []
    for s in range(warmup + steps):
        o = pkg.psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, pt.depth, seed=tin.seed,
                                    step=s)
        n_all.append(o["accept_len"].clone())
        keep_all.append(o["accept_nodes"].clone())
    del tin
    torch.cuda.empty_cache()
    g = torch.Generator(device="cuda").manual_seed(9)
    len0 = torch.randint(0, Lmax - blk + 1, (warmup + steps, b), generator=g, device="cuda",
                         dtype=torch.int32)
    kv = torch.zeros(b, Lmax, KV_ROW_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    moved = 0
    for s in range(warmup, warmup + steps):
        n = n_all[s].cpu()
        k = keep_all[s].cpu()
        for r in range(b):
            moved += int((k[r, :int(n[r])] != torch.arange(int(n[r]), dtype=torch.int32)).sum())
    lens = [len0.clone(), len0.clone()]

    def call(s, phase=0):
        pkg.psispec_kv_commit(kv, blk, n_all[s], lens[phase][s], keep=keep_all[s])

    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(warmup, warmup + steps):
        call(s)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    pkg.timing_enable(True)
    for s in range(warmup, warmup + steps):
        call(s, 1)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    ok = bool((lens[0][warmup:] == len0[warmup:] + torch.stack(n_all[warmup:])).all().item())
    del kv
    torch.cuda.empty_cache()
    k_us = {k: 1e3 * v[0] / max(1, v[1]) for k, v in kern.items()}
    cp_us = k_us.get("kv_commit", 0.0)
    alg = 2 * KV_ROW_BYTES * moved / steps  # bytes per call
    gbs = alg / (cp_us / 1e6) / 1e9 if cp_us > 0 else 0.0
    return dict(workload=f"kv commit: batch {b} lines x {Lmax} positions x {KV_ROW_BYTES} B rows "
                         f"(bf16, 28 layers x K,V x 8 heads x 128), {blk}-position tree blocks, kept "
                         f"paths from tree verifies (N=32, depth<=8, concentrated rows)",
                us_per_call=round(1e3 * ms / steps, 2), lengths_ok=ok,
                moved_rows_per_call=round(moved / steps, 1),
                kernels_avg_us={k: round(v, 2) for k, v in k_us.items()},
                roofline={"bound": "hbm", "kernel": "k_kv_commit", "achieved": round(gbs, 1),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "traffic": read_traffic("kv_commit", "tree"),
                          "bytes_per_launch": int(alg), "avg_launch_us": round(cp_us, 2)})


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, datasheet


def run_lmhead(steps, warmup, torch, pkg, workloads):
    """Time psispec_lmhead_verify on the batch-128, B=8, H=4096, V=151936, rank-16 LoRA workload."""
    preset = workloads.PRESETS["c5"]
    t0 = time.time()
    inp = workloads.make_lmhead(preset, device="cuda", steps=min(steps + warmup, 8))
    torch.cuda.synchronize()
    log(f"c5: generated inputs in {time.time() - t0:.1f}s")
    b, B, H, V, r = preset.batch, preset.B, preset.H, preset.V, preset.r
    ws = torch.empty(pkg.lmhead_workspace_bytes(b, B, H, V, r), dtype=torch.uint8, device="cuda")
    out = dict(accept_len=torch.empty(b, dtype=torch.int32, device="cuda"),
               out_tokens=torch.empty(b, B + 1, dtype=torch.int32, device="cuda"),
               ratios=torch.empty(b, B, dtype=torch.float32, device="cuda"),
               accept_mask=torch.empty(b, dtype=torch.int64, device="cuda"),
               status=torch.empty(b, dtype=torch.int32, device="cuda"))
    acc = torch.zeros(b, dtype=torch.int64, device="cuda")

    def step(s):
        pkg.psispec_lmhead_verify(inp.h_ar, inp.h_draft, inp.W, inp.drafts[s % len(inp.drafts)],
                                  inp.A, inp.Bl, preset.lora_scale, temperature=preset.T,
                                  seed=inp.seed, step=s, workspace=ws, out=out)

    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    committed = 0
    for s in range(warmup, warmup + steps):
        step(s)
        acc += out["accept_len"].to(torch.int64) + 1
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    committed = int(acc.sum().item())
    pkg.timing_enable(True)
    for s in range(warmup, warmup + steps):
        step(s)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    flops = workloads.lmhead_flops(b, B, H, V, r)
    g = kern.get("lmhead_gemm", (0.0, 1))
    gemm_us = 1e3 * g[0] / max(1, g[1])
    achieved = flops / (gemm_us / 1e6) / 1e12
    return dict(workload=f"c5: LM head + linear verify, batch={b} B={B} H={H} V={V} LoRA rank {r}, "
                         f"bf16 MFMA (fp32 accumulate)",
                ms_per_step=round(ms / steps, 4),
                rows_per_s=round(steps * b * B / (ms / 1e3), 1),
                committed_tokens_per_s=round(committed / (ms / 1e3), 1),
                kernels_avg_us={k: round(1e3 * v[0] / max(1, v[1]), 2) for k, v in kern.items()},
                roofline={"bound": "mfma", "kernel": "k_lmhead_gemm", "achieved": round(achieved, 1),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                          "flops_per_launch": flops, "avg_launch_us": round(gemm_us, 2)})


# Sources each measured kernel is built from (kernel, device bodies, shared helpers): a counter
# summary applies only while their hash matches.
KERNEL_SOURCES = {
    "rowstats": ("rows.hip", "rows.h", "internal.h"),
    "rowstats_topp": ("topp.hip", "rows.h", "launch.h", "internal.h"),
    "draft_bounds": ("drafts.hip", "draw.h", "decide.h", "launch.h", "internal.h"),
    "kv_commit": ("kv.hip", "launch.h", "internal.h"),
}


def source_sha(kernel="rowstats"):
    """Hash of the sources the kernel is built from."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "lossless_draft_verification_spec_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernel
    source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_sha(kernel):
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(host, preset, seconds):
    """The oracle as it stands, single-threaded on this host, on the requests of rotation set 0,
    step after step (Philox step 0, 1, ...), for about `seconds` of work."""
    import numpy as np
    import oracle
    import torch

    p = host["p"].detach().cpu()
    q = host["q"].detach().cpu()
    if p.dtype == torch.bfloat16:
        ph = p.view(torch.int16).numpy().view(np.uint16)
        qh = q.view(torch.int16).numpy().view(np.uint16)
    else:
        ph, qh = p.numpy(), q.numpy()
    d = host["d"].cpu().numpy()
    B = preset.B
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        r, step = done % preset.batch, done // preset.batch
        oracle.verify_linear(ph[r:r + 1], qh[r:r + 1], d[r:r + 1], T=preset.T, top_p=preset.top_p,
                             seed=host["seed"], step=step, request_base=r)
        done += 1
    el = time.perf_counter() - t0
    return dict(value=done * B / el, unit="rows/s", cores=1, kind="oracle",
                sample=f"{done} request verifies (x {B} verified rows): the {preset.batch} requests "
                       f"of rotation set 0 over Philox steps 0..{(done - 1) // preset.batch}, "
                       f"one thread, {el:.1f} s")


def copy_calibration(torch):
    n = 512 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requests would shard by request_base with no exchange).", file=sys.stderr)
        sys.exit(2)
    import torch

    import lossless_draft_verification_spec_amd as pkg
    from lossless_draft_verification_spec_amd import workloads

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    pkg.lib()
    if args.workload == "c5":
        print(json.dumps(run_lmhead(args.lmhead_steps, 3, torch, pkg, workloads)), flush=True)
        return
    if args.workload in ("c4", "c4s"):
        print(json.dumps(run_tree(args.tree_steps, 5, torch, pkg, workloads, args.workload)),
              flush=True)
        return
    if args.workload == "sweep":
        batches = [int(x) for x in args.sweep_batches.split(",") if x]
        print(json.dumps(run_sweep(batches, args.sweep_steps, torch, pkg, workloads,
                                   args.sweep_noise, args.sweep_boost)), flush=True)
        return
    if args.workload == "kv":
        print(json.dumps(run_kv(args.kv_steps, 3, torch, pkg, workloads)), flush=True)
        return
    if args.workload == "drafts":
        print(json.dumps(run_drafts(args.draft_steps, 5, torch, pkg, workloads)), flush=True)
        return
    res, host = run_workload(args.workload, args.steps, args.warmup, torch, pkg, workloads)
    pr = res["preset"]
    log(f"{args.workload}: {res['ms_per_step'] * 1e3:.1f} us/step, kernels {res['kernels']}")
    target = None
    if not args.no_target and args.workload != "ns":
        tres, _ = run_workload("ns", args.steps, args.warmup, torch, pkg, workloads)
        rs = tres["kernels"].get("rowstats", {})
        target = dict(workload="ns: linear verify batch=256 B=8 V=151936 bf16, generated as c2",
                      rows_per_s=round(tres["rows_per_s"], 1),
                      committed_tokens_per_s=round(tres["committed_per_s"], 1),
                      ms_per_step=round(tres["ms_per_step"], 4),
                      hbm_gbs_step=round(tres["hbm_gbs_step"], 1),
                      rowstats_avg_us=round(rs.get("avg_us", 0.0), 2),
                      rowstats_gbs=round(tres.get("rowstats_gbs", 0.0), 1),
                      rowstats_frac_of_peak=round(tres.get("rowstats_gbs", 0.0) / HBM_PEAK_GBS, 4),
                      kernels_avg_us={k: round(v["avg_us"], 2) for k, v in tres["kernels"].items()})
        log(f"ns: {tres['ms_per_step'] * 1e3:.1f} us/step, kernels {tres['kernels']}")
    lmhead = None
    if not args.no_lmhead:
        lmhead = run_lmhead(args.lmhead_steps, 3, torch, pkg, workloads)
        log(f"c5: {lmhead['ms_per_step'] * 1e3:.1f} us/step, kernels {lmhead['kernels_avg_us']}")
    tree = None
    if not args.no_tree:
        tree = run_tree(args.tree_steps, 5, torch, pkg, workloads)
        log(f"c4: {tree['ms_per_step'] * 1e3:.1f} us/step, kernels {tree['kernels_avg_us']}")
    drafts = None
    if not args.no_drafts:
        drafts = run_drafts(args.draft_steps, 5, torch, pkg, workloads)
        log(f"drafts: {drafts['ms_per_step'] * 1e3:.1f} us/step, kernels {drafts['kernels_avg_us']}")
    kvc = None
    if not args.no_kv:
        kvc = run_kv(args.kv_steps, 3, torch, pkg, workloads)
        log(f"kv: {kvc['us_per_call']} us/call, kernels {kvc['kernels_avg_us']}")
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(host, pr, args.cpu_seconds)
    rk = res["row_kernel"]
    rs = res["kernels"][rk]
    achieved = res["row_bytes"] / (rs["avg_us"] / 1e6) / 1e9
    traffic = read_traffic(rk, args.workload)
    line = {
        "metric": "verified rows/s + committed tokens/s, HBM GB/s as % of peak (B=8, V=151936)",
        "value": round(res["rows_per_s"], 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: linear verify batch={pr.batch} B={pr.B} "
                               f"V={pr.V} bf16 logits, T={pr.T}, top_p={pr.top_p}",
                   "batch": pr.batch, "B": pr.B, "V": pr.V, "input_dtype": "bf16",
                   "parallelism": "single GPU", "rotation_sets": pr.rotations},
        "committed_tokens_per_s": round(res["committed_per_s"], 1),
        "mean_committed_per_request": round(res["mean_committed"], 4),
        "hbm_gbs_step": round(res["hbm_gbs_step"], 1),
        "hbm_frac_step": round(res["hbm_gbs_step"] / HBM_PEAK_GBS, 4),
        "kernels_avg_us": {k: round(v["avg_us"], 2) for k, v in res["kernels"].items()},
        "roofline": {"bound": "hbm", "kernel": f"k_{rk}", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": res["row_bytes"],
                     "avg_launch_us": round(rs["avg_us"], 2)},
        "cpu_baseline": cpu,
        "target_shape": target,
        "lmhead": lmhead,
        "tree": tree,
        "drafts": drafts,
        "kv_commit": kvc,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
