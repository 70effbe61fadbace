"""Host-side logic of bench.py (no GPU): the one-GPU guard, the algorithmic
byte count behind the roofline and the counter-summary lookup."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_by_hand_fc1():
    # each input read once (B and SFB of non-empty experts only), each output
    # written once: E4M3 D and D_col (valid_m x N/2) plus both scale arrays
    case = synth.make_case("fc1_swiglu_l8", L=3, K=256, N=128, routing=("topk", 200, 2))
    p, a = case.problem, case.arrays
    vm, n, k, L = p["valid_m"], p["n"], p["k"], p["num_groups"]
    nonempty = int((case.counts > 0).sum())
    reads = vm * k + vm * k // 32 + nonempty * n * k + nonempty * n * k // 32 + 4 * vm
    no = n // 2
    writes = 2 * vm * no + vm * no // 32 + no * vm // 32
    assert a["a"].nbytes == vm * k and a["b"].nbytes == L * n * k
    assert bench.algorithmic_bytes(case) == float(reads + writes)


def test_algorithmic_bytes_backward_counts_c_in_and_dprob():
    case = synth.make_case("dswiglu_bf16_l64", L=2, K=64, N=64, routing=("topk", 100, 1))
    p, a = case.problem, case.arrays
    vm, n, k = p["valid_m"], p["n"], p["k"]
    nonempty = int((case.counts > 0).sum())
    reads = 2 * vm * k + nonempty * n * k * 2 + 4 * vm + vm * 2 * n * 2
    writes = vm * 2 * n * 2 + 4 * vm
    assert a["c_in"].nbytes == vm * 2 * n * 2
    assert bench.algorithmic_bytes(case) == float(reads + writes)


def test_profile_lookup_needs_matching_workload_and_kernel(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    f = tmp_path / "t.md"
    monkeypatch.setattr(bench, "PROFILE_FILE", str(f))
    f.write_text(f"kernel_source_sha256_16: {h}\n\n```\n"
                 "workload=fc1_swiglu_l64 hbm_bytes_per_launch=1.5e9 sclk_mhz=1875.0 mfma_busy_frac=0.57\n"
                 "workload=fc1_swiglu_l64:rowmajor hbm_bytes_per_launch=1.6e9\n```\n")
    assert bench.read_profile("fc1_swiglu_l64") == {"hbm_bytes_per_launch": 1.5e9, "sclk_mhz": 1875.0,
                                                    "mfma_busy_frac": 0.57}
    assert bench.read_profile("fc1_swiglu_l64:rowmajor") == {"hbm_bytes_per_launch": 1.6e9}
    assert bench.read_profile("fc1_swiglu_l8") is None
    f.write_text("kernel_source_sha256_16: 0000000000000000\n"
                 "workload=fc1_swiglu_l64 hbm_bytes_per_launch=1.5e9\n")
    assert bench.read_profile("fc1_swiglu_l64") is None


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "k.h"
    src.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["k.h"])
    h0 = bench.kernel_source_hash()
    src.write_text("/* header */\nint f(int x) {\n    return x + 1;   // another comment\n}\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.kernel_source_hash() != h0
