"""Host logic of bench.py that needs no GPU: the roofline arithmetic, how the two measurements of
the ceilings combine, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_fractions():
    r = bench.roofline_hbm("k", 8e9, 1e6, {"hbm_read_gbs": 7000.0})  # 8 GB in 1 s
    assert r["bound"] == "hbm" and r["achieved"] == 8.0 and r["frac"] == round(8.0 / 8000.0, 4)
    assert r["peak_measured"] == 7000.0 and r["frac_measured"] == round(8.0 / 7000.0, 4)
    m = bench.roofline_mfma("g", 2.5e15, 1e6, None)  # 2.5 PFLOP in 1 s
    assert m["bound"] == "mfma" and m["achieved"] == 2500.0 and m["frac"] == 1.0
    assert "frac_measured" not in m


def test_ceilings_take_the_better_run_and_refresh_every_fraction():
    a = {"hbm_read_gbs": 6850.0, "hbm_read_us": 627.0, "mfma_bf16_tflops": 2436.0,
         "mfma_us": 3526.0, "method": "m"}
    b = {"hbm_read_gbs": 7150.0, "hbm_read_us": 600.7, "mfma_bf16_tflops": 2400.0,
         "mfma_us": 3579.0, "method": "m"}
    p = bench.best_peaks(a, b)
    assert p["hbm_read_gbs"] == 7150.0 and p["hbm_read_us"] == 600.7  # the second run read faster
    assert p["mfma_bf16_tflops"] == 2436.0 and p["mfma_us"] == 3526.0  # the first issued faster
    assert p["hbm_read_gbs_runs"] == [6850.0, 7150.0]
    leg = {"roofline": bench.roofline_hbm("k", 6945.9e3, 1.0, a), "hbm_gbs_step": 5060.0,
           "hbm_frac_step_measured": 5060.0 / 6850.0}
    assert leg["roofline"]["frac_measured"] > 1.0  # against the low ceiling
    bench.apply_peaks(leg, p)
    assert leg["roofline"]["peak_measured"] == 7150.0
    assert leg["roofline"]["frac_measured"] == round(6945.9 / 7150.0, 4)
    assert leg["hbm_frac_step_measured"] == round(5060.0 / 7150.0, 4)
    g = {"roofline": bench.roofline_mfma("g", 1.3e15, 1e6, a)}
    bench.apply_peaks(g, p)
    assert g["roofline"]["frac_measured"] == round(1300.0 / 2436.0, 4)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
