"""Throughput of the grouped block-scaled GEMM + fused epilogue on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also LIST]
                    [--no-cpu-baseline] [--no-cold] [--profile-launches N]

A step is one launch of the whole hot path (grouped MXFP8 GEMM, SwiGLU over
32-column pairs, gating, FP8 row + column quantisation with E8M0 scales) over
the FC1 + SwiGLU workload at L = 64 experts: 16384 tokens routed top-6
uniformly (98304 routed rows, each expert padded to a multiple of 128 rows),
K = 2048, N = 2816 (44 linear/gate pairs of 32 columns), MXFP8 E4M3 operands
with E8M0 scales per 32 K-elements, passed in the library's K-block plane
layout (laid out on the device before the timed region).  The same line also
reports the other workloads of `--also` (the 8-expert FC1 + SwiGLU workload,
the other configurations, the row-major scale layout, discrete weights),
which run first.  Inputs are synthetic and already resident in HBM.  Rank 0
prints one JSON line.  Per workload: the mean per launch over the timed
window (HIP events on the launch stream around every launch) with its
median, min and max, and the mean after a 1 GiB cache flush (cold).

`value` is TFLOP/s over routed rows (2 * routed * N * K per step, padding
excluded).  `roofline` compares the kernel's achieved rate (HIP events on the
launch stream) with the dense MXFP8 MFMA peak; `traffic`, the core clock
under the kernel (and the roofline fraction at that clock) and the MFMA-busy
fraction come from the committed rocprofv3 counter summary when it was taken
on the current kernel source, else they are left out (traffic null).
`cpu_baseline` is the C++ float64 oracle on the host cores.
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
PREWARM = 40                  # untimed launches before the first measured workload
KERNEL_SOURCES = ["moe_grouped_block_amd/csrc/grouped_gemm.h", "moe_grouped_block_amd/csrc/moegg_kernels.hip",
                  "moe_grouped_block_amd/csrc/inst_e4m3.hip", "moe_grouped_block_amd/csrc/inst_e2m1.hip",
                  "moe_grouped_block_amd/csrc/inst_bf16.hip", "moe_grouped_block_amd/csrc/inst_e5m2.hip",
                  "moe_grouped_block_amd/csrc/moegg_internal.h"]
PROFILE_FILE = "profiles/grouped_gemm_counters_bench_workloads.md"


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


def read_profile(workload: str):
    """Counter-derived figures of one workload from the committed rocprofv3
    summary (HBM bytes per launch, the core clock while its kernel ran, the
    MFMA-busy fraction), if that summary was taken on the current kernel
    source; else None."""
    path = os.path.join(ROOT, PROFILE_FILE)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m_hash or m_hash.group(1) != kernel_source_hash():
        return None
    for m in re.finditer(r"^workload=(\S+)((?: [a-z_]+=\S+)*)\s*$", text, re.M):
        if m.group(1) == workload:
            return {k: float(v) for k, v in (kv.split("=") for kv in m.group(2).split())}
    return None


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
    """The C++ float64 oracle as it stands (plain loops, OpenMP over rows) on
    the host cores, on the first `rows_n` rows of the workload.  If the C++
    oracle cannot be loaded or built on this host, the numpy oracle is timed
    instead (its own threads, on 2.5x the rows) and the sample says so."""
    import numpy as np
    p = case.problem
    try:
        from oracle import cxx
        cxx.lib()
        run, cores, what = cxx.grouped_gemm, cxx.threads(), "C++ float64 oracle"
        what += f" (dequantise, GEMM, SwiGLU, FP8 row and column quantisation) on {cores} OpenMP threads"
    except Exception as e:                     # no compiler / library on this host
        import oracle
        try:
            from threadpoolctl import threadpool_info
            cores = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        except Exception:
            cores = os.cpu_count() or 1
        rows_n = int(rows_n * 2.5)
        run, what = oracle.grouped_gemm, f"numpy float64 oracle (the C++ one failed to load: {str(e)[:80]})"
    rows_n = min(rows_n, p["valid_m"])
    rows = np.arange(rows_n)
    routed = int(case.row_valid[:rows_n].sum())
    t0 = time.perf_counter()
    run(p, case.arrays, rows)
    dt = time.perf_counter() - t0
    flops = 2.0 * routed * p["n"] * p["k"]
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"rows [0, {rows_n}) of the workload ({routed} routed rows), one pass of the {what}: "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed launches of the headline before its timed window")
    ap.add_argument("--workload", default="fc1_swiglu_l64")
    ap.add_argument("--also", default="fc2_gating_l64_zipf,srelu_tanh_fp4_l32,dswiglu_bf16_l64,"
                    "fc1_swiglu_l64:discrete,fc1_swiglu_l64:rowmajor,fc1_swiglu_l8,quant_gating_l4,"
                    "fc1_geglu_e5m2_l8,dswiglu_mxfp8_l64,dsrelu_mxfp8_l32,dgeglu_mxfp8_l64",
                    help="comma list of extra workloads to time (before the headline; the small ones after "
                         "long ones, so that the host has queued far ahead of the GPU and their launches run "
                         "back to back instead of at the host's launch rate).  Scales are passed as "
                         "K-block planes (sf_layout KPLANES) unless a ':rowmajor' suffix asks for the row-major "
                         "(rows, K/32) layout; a ':discrete' suffix passes the expert weights as per-expert "
                         "allocations (b_ptrs / sfb_ptrs)")
    ap.add_argument("--cpu-rows", type=int, default=49152, help="rows of the oracle CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true", help="skip the launches after an L2/MALL flush")
    ap.add_argument("--profile-launches", type=int, default=0,
                    help="profiling mode: launch every workload (the --also list, then --workload) this "
                         "many times back to back, untimed, and print the order (for rocprofv3 passes)")
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

    def prepare(name):
        """Upload one workload (inputs resident in HBM, scales laid out as the
        workload's mode asks) and return (case, launch function, tensors)."""
        base, *modes = name.split(":")
        if set(modes) - {"discrete", "rowmajor"}:
            raise SystemExit(f"unknown workload mode in {name!r}")
        case = synth.make_case(base)
        layout = "row_major" if "rowmajor" in modes else "kplanes"
        p = dict(case.problem, sf_layout=layout)
        dev = pl.to_device(case.arrays, sf_layout=layout, k=p["k"])
        outs = pl.empty_outputs(p)
        keep = None
        if "discrete" in modes:
            ptrs, keep = pl.discrete_weights(p, case.arrays, seed=case.seed, sf_layout=layout)
            del dev["b"]
            dev.pop("sfb", None)
            tensors = {**pl.inputs_for(p, dev, discrete=ptrs), **outs}
        else:
            tensors = {**pl.inputs_for(p, dev), **outs}
        stream = torch.cuda.current_stream()
        prob_s, args_s = mg.make_problem(p), mg.make_args(tensors)
        handle = stream.cuda_stream

        def step():
            st = mg.moegg_run(prob_s, args_s, handle)
            if st != 0:
                raise mg.MoeggError(st, mg.moegg_last_error())
        torch.cuda.synchronize()
        return case, step, (dev, outs, tensors, keep)

    names = [x for x in args.also.split(",") if x] + [args.workload]
    if args.profile_launches > 0:
        for name in names:
            _, step, held = prepare(name)
            for _ in range(args.profile_launches):
                step()
            torch.cuda.synchronize()
            del held
            torch.cuda.empty_cache()
        print(json.dumps({"profile_order": names, "launches": args.profile_launches}), flush=True)
        return

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if not args.no_cold else None   # 1 GiB

    def enqueue(name, prepared, steps, warmup, cold):
        """Enqueue one workload's warmup launches, its timed launches (an event
        before every launch and one after the last, on the launch stream) and
        its cold launches (each after a 1 GiB write that evicts L2 and MALL),
        without waiting for any of it: the host never leaves the GPU idle
        between workloads.  Returns what `collect` reads after the stream has
        run."""
        case, step, held = prepared
        stream = torch.cuda.current_stream()
        for _ in range(warmup):
            step()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for i in range(steps):
            ev[i].record(stream)
            step()
        ev[steps].record(stream)
        cold_ev = []
        if cold:
            for _ in range(10):
                flush.zero_()
                a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a0.record(stream)
                step()
                a1.record(stream)
                cold_ev.append((a0, a1))
        return {"case": case, "name": name, "ev": ev, "cold_ev": cold_ev, "held": held}

    def collect(q):
        ev, steps = q["ev"], len(q["ev"]) - 1
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        ms = ev[0].elapsed_time(ev[steps]) / steps
        case = q["case"]
        res = {"case": case, "name": q["name"], "ms": ms, "tflops": case.flops / (ms * 1e-3) / 1e12,
               "ms_median": per[len(per) // 2], "ms_min": per[0], "ms_max": per[-1]}
        if q["cold_ev"]:
            cl = sorted(a0.elapsed_time(a1) for a0, a1 in q["cold_ev"])
            res["cold_ms"] = sum(cl) / len(cl)
            res["cold_ms_median"] = cl[len(cl) // 2]
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
        prof = read_profile(r["name"])
        if prof and prof.get("sclk_mhz"):
            # the core clock under this kernel (rocprofv3 counters: GPU cycles per
            # XCD over the dispatch time) and the MFMA roofline scaled to it (the
            # HBM roofline does not move with the core clock)
            t_m_clk = t_m * NOMINAL_SCLK_MHZ / prof["sclk_mhz"]
            d["sclk_mhz"] = round(prof["sclk_mhz"], 1)
            d["frac_roofline_at_sclk"] = round(max(t_m_clk, t_h) / (r["ms"] * 1e-3), 4)
        if prof and prof.get("mfma_busy_frac"):
            d["mfma_busy_frac"] = prof["mfma_busy_frac"]
        if prof and prof.get("hbm_bytes_per_launch"):
            d["traffic"] = prof["hbm_bytes_per_launch"]
        if "cold_ms" in r:
            d["cold_ms_per_launch"] = round(r["cold_ms"], 5)
            d["cold_ms_median"] = round(r["cold_ms_median"], 5)
            d["cold_frac_roofline"] = round(max(t_m, t_h) / (r["cold_ms"] * 1e-3), 4)
        return d

    # Every workload is generated and uploaded first; then all of them are
    # enqueued back to back on one stream, the headline last, and the host
    # waits once.  After any idle gap, even of a few milliseconds, the GPU's
    # power management lets a few launches run above the sustained clock,
    # then throttles below it and settles over about 30 launches; with the
    # stream never idle, the headline's window measures the sustained state
    # that a long training run sees.  The first workload would still meet
    # that transient: PREWARM untimed launches of the headline go first.
    prepared = [prepare(name) for name in names]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(PREWARM):
        prepared[-1][1]()
    queued = []
    for i, name in enumerate(names):
        last = i == len(names) - 1
        queued.append(enqueue(name, prepared[i], args.steps if last else max(args.steps, 20),
                              args.warmup if last else max(args.warmup, 10), not args.no_cold))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del prepared
    results = [collect(q) for q in queued]
    del queued
    torch.cuda.empty_cache()
    also = {name: summary(r) for name, r in zip(names[:-1], results[:-1])}
    main_res = results[-1]
    case, ms, value = main_res["case"], main_res["ms"], main_res["tflops"]
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
            "frac": round(achieved / pk, 4), "traffic": hs.get("traffic"),
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
        "wall_s_all_workloads": round(wall, 3),
    }
    line["config"]["sf_layout"] = "kplanes"
    for k in ("sclk_mhz", "mfma_busy_frac", "cold_ms_per_launch", "cold_ms_median", "cold_frac_roofline"):
        if k in hs:
            line[k] = hs[k]
    if also:
        line["also"] = also
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_rows)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
