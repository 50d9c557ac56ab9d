#!/usr/bin/env python3
"""Benchmark of the Psi-Spec verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one psispec_verify_linear call over one batch of synthetic logits: the HBM pass over
every p and q row, the nucleus pass when top-p is on, the accept test and first-rejection scan, and
the fp64 final draw.  The headline workload is the batch-64, B=8, V=151,936 bf16 block (Zipf-boosted
N(0, 3^2) target logits, draft noise sigma in {0.3, 1, 2} per request, T = 1); rotation sets that
together exceed the 256 MB last-level cache are cycled so every step reads its rows from HBM, and
each step has its own drafted tokens and Philox step.  Inputs are resident in HBM before timing.

One JSON line is printed.  `value` is verified rows/s (batch*B per step) over the K timed steps;
beside it committed tokens/s, the per-call device time (median, p10, p90 over --calls timed calls)
and the roofline of the dominant kernel.  Every roofline gives the achieved rate against the
datasheet peak and against the peak measured on this GPU at the start of the run (a 16-byte
nontemporal read sweep over 4 GiB; back-to-back bf16 MFMAs with no memory traffic); kernel times
come from start/stop events that each kernel's dispatch records (the library's timing mode), the
same quantity a rocprofv3 kernel trace reports.  Further legs, each with its own statistics and
roofline: the batch-256 B=8 shape (`target_shape`), the top-p config (`c3`: batch 256, B=16,
T=0.7, top-p 0.95), the 4-token fp32 config (`c1`: latency only), the 32-node trees with chosen
(`tree`) and sampled (`tree_sampled`) candidates, the LM head + verify (`lmhead`: batch 128, B=8,
H=4096, rank-16 LoRA, MFMA roofline), the drafting step (`drafts`), the KV commit after tree
verifies (`kv_commit`), and the oracle timed on the host cores (`cpu_baseline`: one thread and
request-sharded over the cores it may use).
`--workload c2|ns|c3|c1|c4|c4s|c5|drafts|kv|peaks` prints that leg's line alone (for profiling);
`--workload sweep` prints the linear-vs-tree batch sweep (batch 1..256).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, datasheet
MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix cores, datasheet
PROFILES = os.path.join(ROOT, "profiles")
TIMER = ("mean kernel time over the timed launches, from start/stop events recorded by each "
         "kernel's dispatch (hipExtLaunchKernelGGL) on the call's stream")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--calls", type=int, default=60,
                    help="calls timed one by one for the median / p10 / p90 of every leg")
    ap.add_argument("--workload", default="all",
                    choices=["all", "c2", "ns", "c3", "c1", "c4", "c4s", "c5", "drafts", "kv",
                             "sweep", "peaks"])
    ap.add_argument("--sweep-batches", default="1,2,4,8,16,32,64,128,256",
                    help="batch sizes of the linear-vs-tree sweep")
    ap.add_argument("--sweep-steps", type=int, default=40)
    ap.add_argument("--sweep-noise", type=float, default=1.0,
                    help="draft noise sigma of the sweep (draft = target + N(0, sigma^2))")
    ap.add_argument("--sweep-boost", type=float, default=1.0,
                    help="Zipf boost scale of the sweep's target rows (2: concentrated rows)")
    ap.add_argument("--leg-steps", type=int, default=100, help="timed steps of the other legs")
    ap.add_argument("--lmhead-steps", type=int, default=30)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for counter scaling)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------
# timing
# ------------------------------------------------------------------------------------------------
def measure(torch, pkg, call, steps, warmup, ncalls):
    """Time `call(s)` (one library call of step s; returns its accept_len or None):
    A: `steps` calls back to back between two events (the throughput of the timed region);
    B: `ncalls` calls, each between its own two events (per-call median / p10 / p90);
    C: `steps` calls with the library's kernel timing on (mean time per kernel).
    Returns dict(ms_per_step, committed (sum of accept_len + 1 over phase A), call_us, kernels_us,
    kernel_launches)."""
    for s in range(warmup):
        call(s)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    accs = []
    ev0.record()
    for s in range(warmup, warmup + steps):
        a = call(s)
        if a is not None:
            accs.append(a)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1)
    committed = int(sum(int((a.to(torch.int64) + 1).sum().item()) for a in accs)) if accs else 0
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(ncalls)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        call(warmup + i % max(1, steps))
        e1.record()
    torch.cuda.synchronize()
    per = sorted(1e3 * e0.elapsed_time(e1) for e0, e1 in evs)

    def q(f):
        return per[min(len(per) - 1, int(round(f * (len(per) - 1))))]

    call_us = dict(median=round(q(0.5), 2), p10=round(q(0.1), 2), p90=round(q(0.9), 2),
                   mean=round(sum(per) / len(per), 2), n=len(per))
    pkg.timing_enable(True)
    for s in range(warmup, warmup + steps):
        call(s)
    kern = pkg.timing_read()
    pkg.timing_enable(False)
    return dict(ms_per_step=ms / steps, committed=committed, call_us=call_us,
                kernels_us={k: 1e3 * v[0] / max(1, v[1]) for k, v in kern.items()},
                kernel_launches={k: v[1] for k, v in kern.items()})


def roofline_hbm(kernel, nbytes, us, peaks, traffic=None):
    gbs = nbytes / (us / 1e6) / 1e9 if us > 0 else 0.0
    r = {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
         "bytes_per_launch": int(nbytes), "avg_launch_us": round(us, 2), "timer": TIMER}
    if peaks and peaks.get("hbm_read_gbs"):
        r["peak_measured"] = peaks["hbm_read_gbs"]
        r["frac_measured"] = round(gbs / peaks["hbm_read_gbs"], 4)
    return r


def roofline_mfma(kernel, flops, us, peaks, traffic=None):
    tf = flops / (us / 1e6) / 1e12 if us > 0 else 0.0
    r = {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
         "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
         "flops_per_launch": flops, "avg_launch_us": round(us, 2), "timer": TIMER}
    if peaks and peaks.get("mfma_bf16_tflops"):
        r["peak_measured"] = peaks["mfma_bf16_tflops"]
        r["frac_measured"] = round(tf / peaks["mfma_bf16_tflops"], 4)
    return r


# ------------------------------------------------------------------------------------------------
# measured peaks
# ------------------------------------------------------------------------------------------------
def measure_peaks(torch, pkg):
    """The HBM read bandwidth of 16-byte nontemporal loads: the best rate over the whole 4 GiB buffer
    (16x the last-level cache; three segment sizes per workgroup, three launches each) and over
    its four 1 GiB quarters read in turn (a quarter is read again only after the three others, so
    the last-level cache holds none of it; four segment sizes, each quarter once); and the bf16
    MFMA issue rate with no memory traffic, the best of five launches (library kernel timing)."""
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sweep = (256 * 16, 256 * 64, 256 * 128)  # 1 MiB, 256 KiB and 128 KiB per workgroup
    qbytes = nbytes // 4
    qsweep = (qbytes >> 18, qbytes >> 17, qbytes >> 16, qbytes >> 15)  # 256 .. 32 KiB per workgroup
    out = torch.empty(max(max(sweep), max(qsweep)), dtype=torch.int32, device="cuda")
    pkg.peak_read(buf, out, sweep[0])
    torch.cuda.synchronize()
    best_gbs = 0.0

    def timed(view, blocks):
        pkg.timing_enable(True)
        pkg.peak_read(view, out, blocks)
        k = pkg.timing_read()
        pkg.timing_enable(False)
        us = 1e3 * k["peak_read"][0] / max(1, k["peak_read"][1])
        return view.numel() / (us / 1e6) / 1e9

    for blocks in sweep:
        for _ in range(3):
            best_gbs = max(best_gbs, timed(buf, blocks))
    for blocks in qsweep:
        for q in range(4):
            best_gbs = max(best_gbs, timed(buf[q * qbytes:(q + 1) * qbytes], blocks))
    best_read = nbytes / (best_gbs * 1e9) * 1e6  # the best rate as the time of the whole buffer
    del buf
    torch.cuda.empty_cache()
    mblocks, iters = 256 * 4, 4000
    mout = torch.empty(mblocks * 256, dtype=torch.float32, device="cuda")
    pkg.peak_mfma(iters, mout, mblocks)
    torch.cuda.synchronize()
    best_mfma = None
    for _ in range(5):
        pkg.timing_enable(True)
        pkg.peak_mfma(iters, mout, mblocks)
        k = pkg.timing_read()
        pkg.timing_enable(False)
        us = 1e3 * k["peak_mfma"][0] / max(1, k["peak_mfma"][1])
        best_mfma = us if best_mfma is None else min(best_mfma, us)
    flops = mblocks * 4 * iters * 16 * 32768 * 1.0
    return dict(hbm_read_gbs=round(nbytes / (best_read / 1e6) / 1e9, 1),
                hbm_read_bytes=nbytes, hbm_read_us=round(best_read, 2),
                mfma_bf16_tflops=round(flops / (best_mfma / 1e6) / 1e12, 1),
                mfma_flops=flops, mfma_us=round(best_mfma, 2),
                datasheet={"hbm_gbs": HBM_PEAK_GBS, "mfma_bf16_tflops": MFMA_BF16_PEAK_TFLOPS},
                method="read: every 16-byte word of a 4 GiB buffer once, nontemporal 16-byte "
                       "loads, 4096, 16384 or 32768 workgroups of 256 threads each streaming a "
                       "contiguous 1 MiB, 256 KiB or 128 KiB segment, 8 loads in flight per "
                       "thread, best of 3 launches of each; also each 1 GiB quarter in turn in "
                       "256, 128, 64 or 32 KiB segments; the best rate of all; "
                       "mfma: 1024 workgroups of 4 waves, "
                       "4000 x 16 independent v_mfma_f32_32x32x16_bf16 per wave, no memory "
                       "traffic, best of 5 launches")


def best_peaks(a, b):
    """The better of two measurements of the ceilings (each figure on its own), with both kept."""
    out = dict(a)
    for key, us_key in (("hbm_read_gbs", "hbm_read_us"), ("mfma_bf16_tflops", "mfma_us")):
        out[key + "_runs"] = [a[key], b[key]]
        if b[key] > a[key]:
            out[key], out[us_key] = b[key], b[us_key]
    out["method"] = a["method"] + "; measured before the legs and again after them, the better kept"
    return out


def apply_peaks(leg, peaks):
    """Re-derive a leg's measured-peak fractions from the final ceilings."""
    rf = leg.get("roofline")
    if rf and rf.get("bound") == "hbm":
        rf["peak_measured"] = peaks["hbm_read_gbs"]
        rf["frac_measured"] = round(rf["achieved"] / peaks["hbm_read_gbs"], 4)
    elif rf and rf.get("bound") == "mfma":
        rf["peak_measured"] = peaks["mfma_bf16_tflops"]
        rf["frac_measured"] = round(rf["achieved"] / peaks["mfma_bf16_tflops"], 4)
    if leg.get("hbm_gbs_step") is not None and "hbm_frac_step_measured" in leg:
        leg["hbm_frac_step_measured"] = round(leg["hbm_gbs_step"] / peaks["hbm_read_gbs"], 4)


# ------------------------------------------------------------------------------------------------
# legs
# ------------------------------------------------------------------------------------------------
def run_linear(name, steps, warmup, ncalls, torch, pkg, workloads, peaks):
    """Time psispec_verify_linear on a linear preset (rotation sets cycled so every step reads its
    rows from HBM)."""
    preset = workloads.PRESETS[name]
    R = preset.rotations
    per_rot = (steps + warmup + R - 1) // R + 1
    t0 = time.time()
    sets = [workloads.make_linear(preset, device="cuda", rotation=i, steps=per_rot) for i in range(R)]
    torch.cuda.synchronize()
    log(f"{name}: generated {R} rotation sets in {time.time() - t0:.1f}s")
    b, B, V = preset.batch, preset.B, preset.V
    elem = 2 if preset.dtype == torch.bfloat16 else 4
    dt = pkg.PSISPEC_BF16 if elem == 2 else pkg.PSISPEC_F32
    ws = torch.empty(pkg.linear_workspace_bytes(b, B, V, dt), dtype=torch.uint8, device="cuda")
    nout = 8
    # accept_len of step s goes to acc_all[s] (no extra copy in the timed region)
    acc_all = torch.zeros(warmup + steps, b, dtype=torch.int32, device="cuda")
    outs = [dict(out_tokens=torch.empty(b, B + 1, dtype=torch.int32, device="cuda"),
                 ratios=torch.empty(b, B, dtype=torch.float32, device="cuda"),
                 accept_mask=torch.empty(b, dtype=torch.int64, device="cuda"),
                 status=torch.empty(b, dtype=torch.int32, device="cuda")) for _ in range(nout)]
    nd = len(sets[0].drafts)

    def call(s):
        inp = sets[s % R]
        d = inp.drafts[(s // R) % nd]
        o = dict(outs[s % nout], accept_len=acc_all[s])
        pkg.psispec_verify_linear(inp.p, inp.q, d, temperature=preset.T, top_p=preset.top_p,
                                  seed=inp.seed, step=s, workspace=ws, out=o)
        return None

    m = measure(torch, pkg, call, steps, warmup, ncalls)
    # every call of step s gives the same outputs: the count of the timed steps
    m["committed"] = int((acc_all[warmup:warmup + steps].to(torch.int64) + 1).sum().item())
    host = dict(p=sets[0].p, q=sets[0].q, d=sets[0].drafts[0], seed=sets[0].seed)
    del sets
    torch.cuda.empty_cache()
    row_bytes = b * (2 * B + 1) * V * elem
    rk = "rowstats" if "rowstats" in m["kernels_us"] else "rowstats_topp"
    ms = m["ms_per_step"]
    res = dict(workload=f"{name}: linear verify batch={b} B={B} V={V} "
                        f"{'bf16' if elem == 2 else 'fp32'} logits, T={preset.T}, "
                        f"top_p={preset.top_p}",
               batch=b, B=B, V=V, steps=steps,
               ms_per_step=round(ms, 5),
               rows_per_s=round(b * B / (ms / 1e3), 1),
               committed_tokens_per_s=round(m["committed"] / (ms * steps / 1e3), 1),
               mean_committed_per_request=round(m["committed"] / (steps * b), 4),
               call_us=m["call_us"],
               hbm_gbs_step=round(workloads.algorithmic_bytes_linear(b, B, V, elem) / (ms / 1e3)
                                  / 1e9, 1),
               kernels_avg_us={k: round(v, 2) for k, v in m["kernels_us"].items()})
    res["hbm_frac_step"] = round(res["hbm_gbs_step"] / HBM_PEAK_GBS, 4)
    if peaks and peaks.get("hbm_read_gbs"):
        res["hbm_frac_step_measured"] = round(res["hbm_gbs_step"] / peaks["hbm_read_gbs"], 4)
    if name != "c1":
        res["roofline"] = roofline_hbm(f"k_{rk}", row_bytes, m["kernels_us"].get(rk, 0.0), peaks,
                                       read_traffic(rk, name))
    else:
        res["roofline"] = None
        res["note"] = "1,152 bytes per call: launch-latency-bound, no roofline claim"
    return res, host


def run_tree(name, steps, warmup, ncalls, torch, pkg, workloads, peaks):
    """Time psispec_verify_tree on the 8-request, 32-node, V=151936 fp32 trees (rotation sets
    exceeding the last-level cache); HBM roofline of the row pass over the N+1 node rows (and the
    N+1 draft rows for `c4s`, whose candidates are drawn from the draft and verified by recursive
    rejection)."""
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
    # the drafter's fan-out, known to the caller from its branching schedule: passed as the bound on
    # children per node, so that the residual passes for wider nodes are not launched
    fan = 0
    if sampled:
        par = sets[0].parent[0].cpu().tolist()
        fan = max(par.count(v) for v in set(par))

    def call(s):
        inp = sets[s % R]
        o = pkg.psispec_verify_tree(inp.p, inp.parent, inp.node_tokens, preset.depth,
                                    temperature=preset.T, top_p=preset.top_p, seed=inp.seed,
                                    step=s, workspace=ws, q_logits=inp.q if sampled else None,
                                    max_children=fan)
        return o["accept_len"]

    m = measure(torch, pkg, call, steps, warmup, ncalls)
    del sets
    torch.cuda.empty_cache()
    row_bytes = b * (N + 1) * V * elem * (2 if sampled else 1)
    ms = m["ms_per_step"]
    rule = f"candidates drawn from the draft (recursive rejection, at most {fan} children per " \
        "node, given)" if sampled else "top-4 candidates"
    return dict(workload=f"{name}: tree verify batch={b} N={N} nodes depth<={preset.depth} V={V} "
                         f"{'bf16' if elem == 2 else 'fp32'} logits, T={preset.T}, {rule}",
                ms_per_step=round(ms, 5),
                nodes_per_s=round(b * N / (ms / 1e3), 1),
                committed_tokens_per_s=round(m["committed"] / (ms * steps / 1e3), 1),
                mean_committed_per_request=round(m["committed"] / (steps * b), 4),
                call_us=m["call_us"],
                kernels_avg_us={k: round(v, 2) for k, v in m["kernels_us"].items()},
                kernel_launches=m["kernel_launches"],
                roofline=roofline_hbm("k_rowstats", row_bytes, m["kernels_us"].get("rowstats", 0.0),
                                      peaks, read_traffic("rowstats", name)))


def run_lmhead(steps, warmup, ncalls, torch, pkg, workloads, peaks):
    """Time psispec_lmhead_verify on the batch-128, B=8, H=4096, V=151936, rank-16 LoRA workload
    (W [H][V], logits never materialised); MFMA roofline of the main matrix-product pass."""
    preset = workloads.PRESETS["c5"]
    t0 = time.time()
    inp = workloads.make_lmhead(preset, device="cuda", steps=min(steps + warmup, 8))
    torch.cuda.synchronize()
    log(f"c5: generated inputs in {time.time() - t0:.1f}s")
    b, B, H, V, r = preset.batch, preset.B, preset.H, preset.V, preset.r
    ws = torch.empty(pkg.lmhead_workspace_bytes(b, B, H, V, r), dtype=torch.uint8, device="cuda")
    acc_all = torch.zeros(warmup + steps, b, dtype=torch.int32, device="cuda")
    out = dict(out_tokens=torch.empty(b, B + 1, dtype=torch.int32, device="cuda"),
               ratios=torch.empty(b, B, dtype=torch.float32, device="cuda"),
               accept_mask=torch.empty(b, dtype=torch.int64, device="cuda"),
               status=torch.empty(b, dtype=torch.int32, device="cuda"))

    def call(s):
        pkg.psispec_lmhead_verify(inp.h_ar, inp.h_draft, inp.W, inp.drafts[s % len(inp.drafts)],
                                  inp.A, inp.Bl, preset.lora_scale, temperature=preset.T,
                                  seed=inp.seed, step=s, workspace=ws,
                                  out=dict(out, accept_len=acc_all[s]))
        return None

    m = measure(torch, pkg, call, steps, warmup, 50)
    m["committed"] = int((acc_all[warmup:warmup + steps].to(torch.int64) + 1).sum().item())
    del inp
    torch.cuda.empty_cache()
    flops = workloads.lmhead_flops(b, B, H, V, r)
    ms = m["ms_per_step"]
    return dict(workload=f"c5: LM head + linear verify, batch={b} B={B} H={H} V={V} LoRA rank {r}, "
                         f"W [H][V] bf16, MFMA with fp32 accumulation, logits never written",
                ms_per_step=round(ms, 5),
                rows_per_s=round(b * B / (ms / 1e3), 1),
                committed_tokens_per_s=round(m["committed"] / (ms * steps / 1e3), 1),
                call_us=m["call_us"],
                kernels_avg_us={k: round(v, 2) for k, v in m["kernels_us"].items()},
                roofline=roofline_mfma("k_lmhead_gemm", flops,
                                       m["kernels_us"].get("lmhead_gemm", 0.0), peaks,
                                       read_traffic("lmhead_gemm", "c5")))


def run_drafts(steps, warmup, ncalls, torch, pkg, workloads, peaks, name="c2"):
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

    def call(s):
        inp = sets[s % R]
        pkg.psispec_sample_drafts(inp.q, ar_logits=inp.p, temperature=preset.T, top_p=preset.top_p,
                                  seed=inp.seed, step=s, flags=F, workspace=ws, out=out)
        return None

    m = measure(torch, pkg, call, steps, warmup, ncalls)
    del sets
    torch.cuda.empty_cache()
    row_bytes = b * B * V * elem  # every sampled row read once
    ms = m["ms_per_step"]
    return dict(workload=f"drafts ({name}): Uno-layout drafting batch={b} B={B} V={V} "
                         f"{'bf16' if elem == 2 else 'fp32'} logits, T={preset.T}, "
                         f"top_p={preset.top_p}",
                ms_per_step=round(ms, 5),
                drafted_tokens_per_s=round(b * B / (ms / 1e3), 1),
                call_us=m["call_us"],
                kernels_avg_us={k: round(v, 2) for k, v in m["kernels_us"].items()},
                roofline=roofline_hbm("k_draft_bounds", row_bytes,
                                      m["kernels_us"].get("draft_bounds", 0.0), peaks,
                                      read_traffic("draft_bounds", name)))


KV_ROW_BYTES = 28 * 2 * 8 * 128 * 2  # one position: 28 layers x (K, V) x 8 KV heads x 128 dims, bf16


def run_kv(steps, warmup, ncalls, torch, pkg, workloads, peaks):
    """Time psispec_kv_commit after tree verifies: batch 256 lines of 160 positions of 114,688-byte
    rows (4.7 GB), 32-position blocks; the kept paths are the accepted nodes of tree verifies of the
    concentrated sweep workload (N=32, depth <= 8, top-4, V=151936 bf16), one set per step, and each
    step has its own line lengths (each call starts from a fresh copy of its step's lengths, a
    4 KB copy that runs before the timed kernels).  HBM roofline of the copy kernel over the bytes
    it must move (each moved row read once and written once)."""
    from dataclasses import replace
    b, Lmax, blk = 256, 160, 32
    pt = replace(workloads.PRESETS["sweep_tree"], boost=2.0)
    tin = workloads.make_tree(pt, device="cuda", batch=b)
    nset = warmup + steps
    n_all, keep_all = [], []
    for s in range(nset):
        o = pkg.psispec_verify_tree(tin.p, tin.parent, tin.node_tokens, pt.depth, seed=tin.seed,
                                    step=s)
        n_all.append(o["accept_len"].clone())
        keep_all.append(o["accept_nodes"].clone())
    del tin
    torch.cuda.empty_cache()
    g = torch.Generator(device="cuda").manual_seed(9)
    len0 = torch.randint(0, Lmax - blk + 1, (nset, b), generator=g, device="cuda",
                         dtype=torch.int32)
    kv = torch.zeros(b, Lmax, KV_ROW_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    moved = 0
    for s in range(warmup, nset):
        n = n_all[s].cpu()
        k = keep_all[s].cpu()
        for r in range(b):
            moved += int((k[r, :int(n[r])] != torch.arange(int(n[r]), dtype=torch.int32)).sum())
    lens = len0.clone()

    def call(s):
        s = s % nset
        lens[s].copy_(len0[s])
        pkg.psispec_kv_commit(kv, blk, n_all[s], lens[s], keep=keep_all[s])
        return None

    m = measure(torch, pkg, call, steps, warmup, ncalls)
    ok = bool((lens[warmup:] == len0[warmup:] + torch.stack(n_all[warmup:])).all().item())
    del kv
    torch.cuda.empty_cache()
    alg = 2 * KV_ROW_BYTES * moved / steps  # bytes per call
    return dict(workload=f"kv commit: batch {b} lines x {Lmax} positions x {KV_ROW_BYTES} B rows "
                         f"(bf16, 28 layers x K,V x 8 heads x 128), {blk}-position tree blocks, kept "
                         f"paths from tree verifies (N=32, depth<=8, concentrated rows)",
                us_per_call=round(1e3 * m["ms_per_step"], 2), lengths_ok=ok,
                moved_rows_per_call=round(moved / steps, 1),
                call_us=m["call_us"],
                kernels_avg_us={k: round(v, 2) for k, v in m["kernels_us"].items()},
                roofline=roofline_hbm("k_kv_commit", alg, m["kernels_us"].get("kv_commit", 0.0),
                                      peaks, read_traffic("kv_commit", "tree")))


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
    the Zipf boost, draft = target + N(0, noise^2)).  Each point cycles rotation sets totalling
    >= 600 MB so every call reads its rows from HBM.  Per point: device time per call, committed
    tokens per call and per second, rows read per call and the row pass's share of HBM peak."""
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


# ------------------------------------------------------------------------------------------------
# counter summaries and the CPU baseline
# ------------------------------------------------------------------------------------------------
# Sources each measured kernel is built from (kernel, device bodies, shared helpers): a counter
# summary applies only while their hash matches.
KERNEL_SOURCES = {
    "rowstats": ("rows.hip", "rows.h", "launch.h", "internal.h"),
    "rowstats_topp": ("topp.hip", "rows.h", "launch.h", "internal.h"),
    "draft_bounds": ("drafts.hip", "draw.h", "decide.h", "launch.h", "internal.h"),
    "kv_commit": ("kv.hip", "launch.h", "internal.h"),
    "lmhead_gemm": ("lmhead.hip", "launch.h", "internal.h"),
}


def source_sha(kernel="rowstats"):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, "lossless_draft_verification_spec_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it matches the current kernel
    source; else None."""
    if kernel not in KERNEL_SOURCES:
        return None
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


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(host, preset, seconds):
    """The oracle as it stands on this host's cores, on the requests of rotation set 0, step after
    step (Philox step 0, 1, ...): one thread for about `seconds`, then the same work sharded by
    request over the cores this process may use (capped at 16, the GPU's share of a shared box),
    one oracle call per request on each thread (the oracle's C code runs without the interpreter
    lock)."""
    import numpy as np
    import oracle
    import torch
    from concurrent.futures import ThreadPoolExecutor

    p = host["p"].detach().cpu()
    q = host["q"].detach().cpu()
    if p.dtype == torch.bfloat16:
        ph = p.view(torch.int16).numpy().view(np.uint16)
        qh = q.view(torch.int16).numpy().view(np.uint16)
    else:
        ph, qh = p.numpy(), q.numpy()
    d = host["d"].cpu().numpy()
    B, nb = preset.B, preset.batch

    def one(k):
        r, step = k % nb, k // nb
        oracle.verify_linear(ph[r:r + 1], qh[r:r + 1], d[r:r + 1], T=preset.T, top_p=preset.top_p,
                             seed=host["seed"], step=step, request_base=r)

    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        one(done)
        done += 1
    el1 = time.perf_counter() - t0
    rate1 = done / el1
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(avail, 16))
    n_multi = max(threads, int(rate1 * seconds * threads * 0.5))  # about seconds/2 if it scales
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(n_multi)))
    el2 = time.perf_counter() - t0
    return dict(value=round(done * B / el1, 1), unit="rows/s", cores=1, kind="oracle",
                sample=f"{done} request verifies (x {B} verified rows) of the batch-{nb}, B={B}, "
                       f"V={preset.V} rows of rotation set 0 over Philox steps 0.."
                       f"{(done - 1) // nb}, one thread, {el1:.1f} s",
                all_cores=dict(value=round(n_multi * B / el2, 1), unit="rows/s", cores=threads,
                               sample=f"{n_multi} request verifies sharded by request over "
                                      f"{threads} threads, {el2:.1f} s"),
                cpu_model=_cpu_model(), nproc=os.cpu_count(), cores_available=avail)


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


# ------------------------------------------------------------------------------------------------
def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (requests would "
              "shard by request_base with no exchange).", file=sys.stderr)
        sys.exit(2)
    import torch

    import lossless_draft_verification_spec_amd as pkg
    from lossless_draft_verification_spec_amd import workloads

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    pkg.lib()
    W, K, C, L = args.warmup, args.steps, args.calls, args.leg_steps
    wl = args.workload
    if wl == "peaks":
        print(json.dumps(measure_peaks(torch, pkg)), flush=True)
        return
    if wl == "sweep":
        batches = [int(x) for x in args.sweep_batches.split(",") if x]
        print(json.dumps(run_sweep(batches, args.sweep_steps, torch, pkg, workloads,
                                   args.sweep_noise, args.sweep_boost)), flush=True)
        return
    single = {
        "c5": lambda: run_lmhead(args.lmhead_steps, 3, C, torch, pkg, workloads, None),
        "c4": lambda: run_tree("c4", L, 5, C, torch, pkg, workloads, None),
        "c4s": lambda: run_tree("c4s", L, 5, C, torch, pkg, workloads, None),
        "drafts": lambda: run_drafts(L, 5, C, torch, pkg, workloads, None),
        "kv": lambda: run_kv(min(L, 50), 3, C, torch, pkg, workloads, None),
        "ns": lambda: run_linear("ns", K, W, C, torch, pkg, workloads, None)[0],
        "c3": lambda: run_linear("c3", L, 5, C, torch, pkg, workloads, None)[0],
        "c1": lambda: run_linear("c1", K, W, C, torch, pkg, workloads, None)[0],
        "c2": lambda: run_linear("c2", K, W, C, torch, pkg, workloads, None)[0],
    }
    if wl in single:
        print(json.dumps(single[wl]()), flush=True)
        return

    t_all = time.time()
    peaks = measure_peaks(torch, pkg)
    log(f"peaks: read {peaks['hbm_read_gbs']} GB/s, bf16 MFMA {peaks['mfma_bf16_tflops']} TFLOP/s")
    res, host = run_linear("c2", K, W, C, torch, pkg, workloads, peaks)
    log(f"c2: {res['ms_per_step'] * 1e3:.1f} us/step, call {res['call_us']}, "
        f"kernels {res['kernels_avg_us']}")
    legs = {}
    for key, fn in (
            ("target_shape", lambda: run_linear("ns", K, W, C, torch, pkg, workloads, peaks)[0]),
            ("c3", lambda: run_linear("c3", L, 5, C, torch, pkg, workloads, peaks)[0]),
            ("c1", lambda: run_linear("c1", K, W, C, torch, pkg, workloads, peaks)[0]),
            ("tree", lambda: run_tree("c4", L, 5, C, torch, pkg, workloads, peaks)),
            ("tree_sampled", lambda: run_tree("c4s", L, 5, C, torch, pkg, workloads, peaks)),
            ("lmhead", lambda: run_lmhead(args.lmhead_steps, 3, C, torch, pkg, workloads, peaks)),
            ("drafts", lambda: run_drafts(L, 5, C, torch, pkg, workloads, peaks)),
            ("kv_commit", lambda: run_kv(min(L, 50), 3, C, torch, pkg, workloads, peaks))):
        legs[key] = fn()
        ms = legs[key].get("ms_per_step", legs[key].get("us_per_call", 0) / 1e3)
        log(f"{key}: {1e3 * ms:.1f} us/call, call {legs[key].get('call_us')}")
    # the ceilings again, on a warm GPU: every measured fraction takes the better of the two runs
    # (a ceiling measured low would overstate them)
    end_peaks = measure_peaks(torch, pkg)
    log(f"peaks at the end: read {end_peaks['hbm_read_gbs']} GB/s, bf16 MFMA "
        f"{end_peaks['mfma_bf16_tflops']} TFLOP/s")
    peaks = best_peaks(peaks, end_peaks)
    for d in (res, *legs.values()):
        apply_peaks(d, peaks)
    pr = workloads.PRESETS["c2"]
    cpu = None if args.no_cpu else cpu_baseline(host, pr, args.cpu_seconds)
    line = {
        "metric": "verified rows/s + committed tokens/s, HBM GB/s as % of peak (B=8, V=151936)",
        "value": res["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"c2: linear verify batch={pr.batch} B={pr.B} V={pr.V} bf16 logits, "
                               f"T={pr.T}, top_p={pr.top_p}",
                   "batch": pr.batch, "B": pr.B, "V": pr.V, "input_dtype": "bf16",
                   "parallelism": "single GPU", "rotation_sets": pr.rotations},
        "committed_tokens_per_s": res["committed_tokens_per_s"],
        "mean_committed_per_request": res["mean_committed_per_request"],
        "call_us": res["call_us"],
        "hbm_gbs_step": res["hbm_gbs_step"],
        "hbm_frac_step": res["hbm_frac_step"],
        "hbm_frac_step_measured": res.get("hbm_frac_step_measured"),
        "kernels_avg_us": res["kernels_avg_us"],
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "peaks_measured": peaks,
        **legs,
        "wall_s": round(time.time() - t_all, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
