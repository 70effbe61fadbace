"""Throughput of the grouped block-scaled GEMM + fused epilogue on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also LIST]
                    [--no-cpu-baseline] [--no-cold] [--no-clock]

A step is one launch of the whole hot path (grouped MXFP8 GEMM, SwiGLU over
32-column pairs, gating, FP8 row + column quantisation with E8M0 scales) over
the FC1 + SwiGLU workload at L = 64 experts: 16384 tokens routed top-6
uniformly (98304 routed rows, each expert padded to a multiple of 128 rows),
K = 2048, N = 2816 (44 linear/gate pairs of 32 columns), MXFP8 E4M3 operands
with E8M0 scales per 32 K-elements.  The same line also reports the 8-expert
FC1 + SwiGLU workload (4096 tokens top-2) and the other workloads of
`--also`, which run first.  Inputs are synthetic and already resident in HBM.
Rank 0 prints one JSON line.  Per workload: the mean per launch over the
timed window (HIP events on the launch stream around every launch) with its
median, min and max; the mean after a 1 GiB cache flush (cold); the core
clock sampled during a further window of launches, and the roofline fraction
at that clock.

`value` is TFLOP/s over routed rows (2 * routed * N * K per step, padding
excluded).  `roofline` compares the kernel's achieved rate (HIP events on the
launch stream) with the dense MXFP8 MFMA peak; `traffic` is read from the
committed rocprofv3 counter summary when it was taken on the current kernel
source, else null.  `cpu_baseline` is the float64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"e4m3": 5000.0, "e5m2": 5000.0, "e2m1x2": 10100.0, "bf16": 2500.0}   # dense MFMA peaks, MI355X
HBM_GBS = 8000.0
NOMINAL_SCLK_MHZ = 2400.0     # the clock at which the MFMA peaks are quoted
KERNEL_SOURCES = ["moe_grouped_block_amd/csrc/grouped_gemm.h", "moe_grouped_block_amd/csrc/moegg_kernels.hip",
                  "moe_grouped_block_amd/csrc/inst_e4m3.hip", "moe_grouped_block_amd/csrc/inst_e2m1.hip",
                  "moe_grouped_block_amd/csrc/inst_bf16.hip", "moe_grouped_block_amd/csrc/inst_e5m2.hip",
                  "moe_grouped_block_amd/csrc/moegg_internal.h"]
TRAFFIC_FILE = "profiles/grouped_gemm_fc1_swiglu_l64_traffic.md"


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code (comments and whitespace removed), so
    that a counter summary stays valid across comment-only edits."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            code = _COMMENT.sub(" ", fh.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it matches
    the current kernel source and workload."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_work = re.search(r"workload:\s*(\S+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_work and m_bytes):
        return None
    if m_hash.group(1) != kernel_source_hash() or m_work.group(1) != workload:
        return None
    return float(m_bytes.group(1))


def algorithmic_bytes(case) -> float:
    """Each input read once (B only for non-empty experts) + each output written once."""
    p, a = case.problem, case.arrays
    nonempty = int((case.counts > 0).sum())
    L = p["num_groups"]
    b_bytes = a["b"].nbytes * nonempty / L + (a["sfb"].nbytes * nonempty / L if "sfb" in a else 0)
    rd = a["a"].nbytes + (a["sfa"].nbytes if "sfa" in a else 0) + b_bytes + a["prob"].nbytes
    rd += a.get("c_in", a["prob"][:0]).nbytes
    vm = p["valid_m"]
    n = p["n"]
    no = {"none": n, "srelu": n, "swiglu": n // 2, "geglu": n // 2, "dswiglu": 2 * n, "dgeglu": 2 * n,
          "dsrelu": n}[p["act"]]
    if p["d_dtype"] == "e4m3":
        wr = 2 * vm * no + vm * no // 32 + no * vm // 32
    else:
        wr = vm * no * 2
    if p["act"] in ("dswiglu", "dsrelu", "dgeglu"):
        wr += vm * 4                      # dprob
    if p.get("c_dtype") == "bf16":
        wr += vm * n * 2
    return float(rd + wr)


def cpu_baseline(case, rows_n):
    """The oracle as it stands on the host cores, on the first `rows_n` rows."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = os.cpu_count() or 1
    p = case.problem
    rows_n = min(rows_n, p["valid_m"])
    rows = np.arange(rows_n)
    routed = int(case.row_valid[:rows_n].sum())
    t0 = time.perf_counter()
    oracle.grouped_gemm(p, case.arrays, rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * routed * p["n"] * p["k"]
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"rows [0, {rows_n}) of the workload ({routed} routed rows), one float64 numpy "
                      f"oracle pass incl. dequantise, GEMM, SwiGLU and FP8 quantisation: {dt:.1f} s"}


class ClockSampler:
    """Median core clock (MHz) of the GPU while a launch window runs, read
    from the driver's metrics through amdsmi in a background thread; None
    where amdsmi is unavailable.  Sampling only reads: it launches nothing."""

    def __init__(self):
        self.h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            vis = os.environ.get("HIP_VISIBLE_DEVICES") or os.environ.get("ROCR_VISIBLE_DEVICES")
            idx = int(vis.split(",")[0]) if vis and vis.split(",")[0].isdigit() and len(hs) > 1 else 0
            self.amdsmi, self.h = amdsmi, hs[min(idx, len(hs) - 1)]
            self.read()
        except Exception as e:   # no driver access: report no clock
            self.h, self.err = None, repr(e)[:200]

    def read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.h)
        v = m.get("current_gfxclks")
        if isinstance(v, (list, tuple)):
            v = [x for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
            if v:
                return float(sum(v)) / len(v)
        for key in ("current_gfxclk", "average_gfxclk_frequency"):
            x = m.get(key)
            if isinstance(x, (int, float)) and 0 < x < 10000:
                return float(x)
        return None

    def during(self, fn):
        """Run fn() while sampling; return (fn's result, median MHz or None, samples)."""
        if self.h is None:
            return fn(), None, 0
        import threading
        vals, stop = [], threading.Event()

        def loop():
            while not stop.is_set():
                try:
                    x = self.read()
                    if x:
                        vals.append(x)
                except Exception:
                    pass
                time.sleep(0.002)
        th = threading.Thread(target=loop, daemon=True)
        th.start()
        try:
            r = fn()
        finally:
            stop.set()
            th.join()
        return r, (float(sorted(vals)[len(vals) // 2]) if vals else None), len(vals)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed launches of the headline before its timed window")
    ap.add_argument("--workload", default="fc1_swiglu_l64")
    ap.add_argument("--also", default="fc1_swiglu_l8,quant_gating_l4,fc2_gating_l64_zipf,srelu_tanh_fp4_l32,"
                    "dswiglu_bf16_l64,fc1_swiglu_l64:discrete,dswiglu_mxfp8_l64,dsrelu_mxfp8_l32,"
                    "fc1_geglu_e5m2_l8,dgeglu_mxfp8_l64",
                    help="comma list of extra workloads to time (before the headline); a ':discrete' suffix "
                         "passes the expert weights as per-expert allocations (b_ptrs / sfb_ptrs)")
    ap.add_argument("--cpu-rows", type=int, default=40960, help="rows of the oracle CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the launches after an L2/MALL flush")
    ap.add_argument("--no-clock", action="store_true", help="skip the clock-sampling window")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy 5 times (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the grouped GEMM is a single-GPU kernel here and "
              "no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import moe_grouped_block_amd as mg
    from moe_grouped_block_amd import plumbing as pl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = 1 << 27
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        torch.cuda.synchronize()
        for _ in range(5):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": True, "bytes_read_per_copy": 4 * n,
                          "bytes_written_per_copy": 4 * n, "copies": 5}), flush=True)
        return
    if not os.path.exists(mg.lib_path):
        from moe_grouped_block_amd import build
        build.build()
    clock = None if args.no_clock else ClockSampler()

    def measure(name, steps, warmup, cold):
        base, _, mode = name.partition(":")
        case = synth.make_case(base)
        p = case.problem
        dev = pl.to_device(case.arrays)
        outs = pl.empty_outputs(p)
        keep = None
        if mode == "discrete":
            ptrs, keep = pl.discrete_weights(p, case.arrays, seed=case.seed)
            del dev["b"]
            dev.pop("sfb", None)
            tensors = {**pl.inputs_for(p, dev, discrete=ptrs), **outs}
        elif mode:
            raise SystemExit(f"unknown workload mode {mode!r}")
        else:
            tensors = {**pl.inputs_for(p, dev), **outs}
        stream = torch.cuda.current_stream()
        prob_s, args_s = mg.make_problem(p), mg.make_args(tensors)
        handle = stream.cuda_stream

        def step():
            st = mg.moegg_run(prob_s, args_s, handle)
            if st != 0:
                raise mg.MoeggError(st, mg.moegg_last_error())

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        # one event before every launch and one after the last, all on the
        # launch stream: launch i takes ev[i] -> ev[i + 1]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        for i in range(steps):
            ev[i].record(stream)
            step()
        ev[steps].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        ms = ev[0].elapsed_time(ev[steps]) / steps
        res = {"case": case, "ms": ms, "wall": wall, "tflops": case.flops / (ms * 1e-3) / 1e12,
               "ms_median": per[len(per) // 2], "ms_min": per[0], "ms_max": per[-1]}
        if clock is not None:
            # a window of back-to-back launches (at least 30 ms) with the clock sampled
            nclk = max(steps, int(30.0 / max(ms, 1e-3)) + 1)

            def window():
                for _ in range(nclk):
                    step()
                torch.cuda.synchronize()
            _, mhz, nsamp = clock.during(window)
            res["sclk_mhz"], res["sclk_samples"] = mhz, nsamp
        if cold:
            flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB > L2 + MALL
            cl = []
            for _ in range(10):
                flush.zero_()
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                step()
                a1.record(stream)
                torch.cuda.synchronize()
                cl.append(a0.elapsed_time(a1))
            res["cold_ms"] = sum(cl) / len(cl)
            res["cold_ms_median"] = sorted(cl)[len(cl) // 2]
            del flush
        del dev, outs, tensors, keep
        torch.cuda.empty_cache()
        return res

    def summary(r):
        c = r["case"]
        peak = PEAK_TFLOPS[c.problem["ab_dtype"]]
        t_m = c.flops / (peak * 1e12)
        t_h = algorithmic_bytes(c) / (HBM_GBS * 1e9)
        padded_flops = 2.0 * c.problem["valid_m"] * c.problem["n"] * c.problem["k"]
        d = {"ms_per_step": round(r["ms"], 5), "ms_median": round(r["ms_median"], 5),
             "ms_min": round(r["ms_min"], 5), "ms_max": round(r["ms_max"], 5),
             "tflops_routed": round(r["tflops"], 2),
             "tflops_padded": round(padded_flops / (r["ms"] * 1e-3) / 1e12, 2),
             "hbm_gbs_algorithmic": round(algorithmic_bytes(c) / (r["ms"] * 1e-3) / 1e9, 1),
             "frac_mfma_peak": round(r["tflops"] / peak, 4),
             "bound": "mfma" if t_m >= t_h else "hbm",
             "frac_roofline": round(max(t_m, t_h) / (r["ms"] * 1e-3), 4),
             "valid_m": c.problem["valid_m"], "routed_rows": c.routed_rows,
             "experts": c.problem["num_groups"]}
        if r.get("sclk_mhz"):
            # the MFMA roofline scaled to the measured clock (the HBM one does not move)
            t_m_clk = t_m * NOMINAL_SCLK_MHZ / r["sclk_mhz"]
            d["sclk_mhz"] = round(r["sclk_mhz"], 1)
            d["frac_roofline_at_sclk"] = round(max(t_m_clk, t_h) / (r["ms"] * 1e-3), 4)
        if "cold_ms" in r:
            d["cold_ms_per_launch"] = round(r["cold_ms"], 5)
            d["cold_ms_median"] = round(r["cold_ms_median"], 5)
            d["cold_frac_roofline"] = round(max(t_m, t_h) / (r["cold_ms"] * 1e-3), 4)
        return d

    # The extra workloads run first: the GPU's power management throttles hard
    # a few launches into sustained load after idle and settles within about
    # 40 launches (25 ms), so the headline's window then measures the
    # sustained state that a long training run sees.
    also = {}
    for name in [x for x in args.also.split(",") if x]:
        r = measure(name, max(args.steps, 20), max(args.warmup, 10), not args.no_cold)
        also[name] = summary(r)
    main_res = measure(args.workload, args.steps, args.warmup, not args.no_cold)
    case, ms, wall, value = main_res["case"], main_res["ms"], main_res["wall"], main_res["tflops"]
    p = case.problem
    hs = summary(main_res)

    peak = PEAK_TFLOPS[p["ab_dtype"]]
    alg_bytes = algorithmic_bytes(case)
    t_mfma = case.flops / (peak * 1e12)
    t_hbm = alg_bytes / (HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    if bound == "mfma":
        achieved, pk, unit = value, peak, "TFLOP/s"
    else:
        achieved, pk, unit = alg_bytes / (ms * 1e-3) / 1e9, HBM_GBS, "GB/s"
    roof = {"bound": bound, "achieved": round(achieved, 2), "peak": pk, "unit": unit,
            "frac": round(achieved / pk, 4), "traffic": read_traffic(args.workload),
            "algorithmic_bytes": alg_bytes, "algorithmic_flops": case.flops}
    if "frac_roofline_at_sclk" in hs:
        roof["sclk_mhz"] = hs["sclk_mhz"]
        roof["frac_at_sclk"] = hs["frac_roofline_at_sclk"]
    line = {
        "metric": "grouped-GEMM TFLOP/s (valid rows) + % MXFP8 MFMA peak, FC1+SwiGLU L=64",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": p["ab_dtype"], "data": "synthetic",
        "config": {"workload": args.workload, "experts": p["num_groups"], "valid_m": p["valid_m"],
                   "routed_rows": case.routed_rows, "n": p["n"], "k": p["k"], "act": p["act"],
                   "d_dtype": p["d_dtype"], "parallelism": "single-gpu"},
        "roofline": roof,
        "pct_mxfp8_peak": round(100.0 * value / PEAK_TFLOPS["e4m3"], 2),
        "ms_per_step_median": hs["ms_median"], "ms_per_step_min": hs["ms_min"], "ms_per_step_max": hs["ms_max"],
        "tflops_padded": hs["tflops_padded"],
        "hbm_gbs_algorithmic": hs["hbm_gbs_algorithmic"],
        "wall_s_timed": round(wall, 4),
    }
    for k in ("sclk_mhz", "cold_ms_per_launch", "cold_ms_median", "cold_frac_roofline"):
        if k in hs:
            line[k] = hs[k]
    if clock is not None and clock.h is None:
        line["sclk_unavailable"] = getattr(clock, "err", "")
    if also:
        line["also"] = also
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
