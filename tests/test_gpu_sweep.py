"""Seeded sweeps over the configuration space, every output against the
oracle: operand family x activation x output format x K-step count x ragged
N x expert count x group alignment (x norm_const and a capped grid, so that
workgroups walk many tiles, in the wider sweep).  The cases are drawn once
from fixed seeds (the same lists on every run), each small enough for the
oracle."""
import numpy as np
import pytest

import synth
from test_gpu_parity import _announce, check_case, run_gpu

mg = pytest.importorskip("moe_grouped_block_amd")

pytestmark = pytest.mark.gpu

BASE = {"none": "quant_gating_l4", "swiglu": "fc1_swiglu_l8", "srelu": "srelu_tanh_fp4_l32",
        "geglu": "fc1_geglu_e5m2_l8", "dswiglu": "dswiglu_mxfp8_l64", "dsrelu": "dsrelu_mxfp8_l32",
        "dgeglu": "dgeglu_mxfp8_l64"}
KSTEP = {"e4m3": 128, "e5m2": 128, "e2m1x2": 256, "bf16": 64}


def draw_cases(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    acts = list(BASE)
    abs_ = list(KSTEP)
    for i in range(n):
        act = acts[i % len(acts)]
        ab = abs_[int(rng.integers(len(abs_)))]
        bwd = act.startswith("d")
        d = "bf16" if (ab == "bf16" and bwd) else ("e4m3" if rng.random() < 0.5 else "bf16")
        c = "bf16" if (not bwd and rng.random() < 0.3) else None
        pair = act in ("swiglu", "geglu")
        n_cols = int(rng.integers(1, 12)) * (64 if pair else 32)
        if d == "e4m3" and act in ("swiglu", "geglu"):
            n_cols = max(n_cols, 64)
        k = int(rng.integers(1, 8)) * KSTEP[ab]
        L = int(rng.integers(1, 10))
        rows = int(rng.integers(1, 500))
        m_al = 256 if rng.random() < 0.25 else 128
        if L >= 2 and rng.random() < 0.5:
            route = dict(routing=("topk", rows, 2), prob=("softmax_picks",))
        else:
            route = dict(routing=("multinomial", rows), prob=("uniform",))
        over = dict(ab=ab, d=d, c=c, L=L, K=k, N=n_cols, m_aligned=m_al, alpha=("uniform", 0.5, 2.0), **route)
        if act == "dswiglu":
            over["beta"] = ("uniform", 0.5, 2.0)
        if ab == "e2m1x2":
            over.update(a_std=1.0, b_std=1.0, clip=6.0)
        if act in ("geglu", "dgeglu"):
            over.update(glu_clamp_min=-2.5, glu_clamp_max=2.0)
        cases.append((f"sweep{i:02d}_{act}_{ab}_{d}", BASE[act], over))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("name,base,over", CASES, ids=[c[0] for c in CASES])
def test_sweep_parity(name, base, over):
    case = synth.make_case(base, seed=5000 + CASES.index((name, base, over)), name=name, **over)
    got = run_gpu(case)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)


def draw_wide_cases(n=48, seed=777):
    """Wider ranges (up to 13 column blocks, 9 K-steps, 11 experts, 1500
    routed rows), norm_const powers of two, and for about half of the cases
    a grid capped at 1-4 workgroups (the moegg_set_grid_limit hook)."""
    rng = np.random.default_rng(seed)
    acts, abs_ = list(BASE), list(KSTEP)
    cases = []
    for i in range(n):
        act = acts[int(rng.integers(len(acts)))]
        ab = abs_[int(rng.integers(len(abs_)))]
        bwd = act.startswith("d")
        d = "bf16" if (ab == "bf16" and bwd) else ("e4m3" if rng.random() < 0.5 else "bf16")
        c = "bf16" if (not bwd and rng.random() < 0.3) else None
        pair = act in ("swiglu", "geglu")
        n_cols = int(rng.integers(1, 14)) * (64 if pair else 32)
        k = int(rng.integers(1, 10)) * KSTEP[ab]
        L = int(rng.integers(1, 12))
        rows = int(rng.integers(1, 1500))
        m_al = 256 if rng.random() < 0.25 else 128
        if L >= 2 and rng.random() < 0.5:
            route = dict(routing=("topk", rows, 2), prob=("softmax_picks",))
        else:
            route = dict(routing=("multinomial", rows), prob=("uniform",))
        over = dict(ab=ab, d=d, c=c, L=L, K=k, N=n_cols, m_aligned=m_al, alpha=("uniform", 0.5, 2.0), **route)
        if act == "dswiglu":
            over["beta"] = ("uniform", 0.5, 2.0)
        if ab == "e2m1x2":
            over.update(a_std=1.0, b_std=1.0, clip=6.0)
        if act in ("geglu", "dgeglu"):
            over.update(glu_clamp_min=-2.5, glu_clamp_max=2.0)
        if rng.random() < 0.3:
            over["norm_const"] = float(2.0 ** int(rng.integers(-3, 4)))
        grid = int(rng.integers(1, 5)) if rng.random() < 0.5 else 0
        cases.append((f"wide{i:02d}_{act}_{ab}_{d}_g{grid}", BASE[act], over, grid))
    return cases


WIDE = draw_wide_cases()


@pytest.mark.parametrize("idx", range(len(WIDE)), ids=[c[0] for c in WIDE])
def test_wide_sweep_parity(idx):
    name, base, over, grid = WIDE[idx]
    case = synth.make_case(base, seed=9000 + idx, name=name, **over)
    print(f"[gpu-case] {name} grid limit {grid or 'none'}", flush=True)
    prev = mg.moegg_set_grid_limit(grid)
    try:
        got = run_gpu(case)
    finally:
        mg.moegg_set_grid_limit(prev)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)


def draw_mixed_cases(n=24, seed=4242):
    """Larger and mixed: up to 64 experts (Zipf routing among them), 6000
    routed rows, 19 column blocks, 11 K-steps; clamp constants and the tanh
    clamp s drawn too; the scales as K-block planes for about 40 % of the MX
    cases, discrete per-expert weights for about a quarter, and a grid capped
    at 1-8 workgroups for half."""
    rng = np.random.default_rng(seed)
    acts, abs_ = list(BASE), list(KSTEP)
    cases = []
    for i in range(n):
        act = acts[int(rng.integers(len(acts)))]
        ab = abs_[int(rng.integers(len(abs_)))]
        bwd = act.startswith("d")
        d = "bf16" if (ab == "bf16" and bwd) else ("e4m3" if rng.random() < 0.5 else "bf16")
        c = "bf16" if (not bwd and rng.random() < 0.3) else None
        pair = act in ("swiglu", "geglu")
        n_cols = int(rng.integers(1, 20)) * (64 if pair else 32)
        k = int(rng.integers(1, 12)) * KSTEP[ab]
        L = int(rng.integers(1, 65))
        rows = int(rng.integers(1, 6000))
        m_al = 256 if rng.random() < 0.25 else 128
        r = rng.random()
        if L >= 6 and r < 0.3:
            route = dict(routing=("topk_zipf", rows, 3, 1.1, 2), prob=("softmax_picks",))
        elif L >= 2 and r < 0.65:
            route = dict(routing=("topk", rows, 2), prob=("softmax_picks",))
        else:
            route = dict(routing=("multinomial", rows), prob=("uniform",))
        over = dict(ab=ab, d=d, c=c, L=L, K=k, N=n_cols, m_aligned=m_al, alpha=("uniform", 0.5, 2.0), **route)
        if act == "dswiglu":
            over["beta"] = ("uniform", 0.5, 2.0)
        if ab == "e2m1x2":
            over.update(a_std=1.0, b_std=1.0, clip=6.0)
        if act in ("geglu", "dgeglu"):
            lo = -float(rng.uniform(0.5, 7))
            hi = float(rng.uniform(0.5, 7))
            over.update(glu_clamp_min=lo, glu_clamp_max=hi)
        if act in ("srelu", "dsrelu"):
            over["s"] = float(rng.choice([0.0, 0.5, 2.0, 8.0, 32.0]))
        if rng.random() < 0.3:
            over["norm_const"] = float(2.0 ** int(rng.integers(-3, 4)))
        grid = int(rng.integers(1, 9)) if rng.random() < 0.5 else 0
        layout = "kplanes" if (ab != "bf16" and rng.random() < 0.4) else "row_major"
        discrete = bool(rng.random() < 0.25)
        tag = f"g{grid}_{'kplanes' if layout == 'kplanes' else 'rows'}{'_discrete' if discrete else ''}"
        cases.append((f"mixed{i:02d}_{act}_{ab}_{d}_{tag}", BASE[act], over, grid, layout, discrete))
    return cases


MIXED = draw_mixed_cases()


@pytest.mark.parametrize("idx", range(len(MIXED)), ids=[c[0] for c in MIXED])
def test_mixed_sweep_parity(idx):
    import torch
    from moe_grouped_block_amd import plumbing as pl
    name, base, over, grid, layout, discrete = MIXED[idx]
    case = synth.make_case(base, seed=20000 + idx, name=name, **over)
    _announce(case)
    print(f"[gpu-case] {name} grid limit {grid or 'none'}, scales {layout}, "
          f"{'discrete' if discrete else 'dense'} weights", flush=True)
    p = dict(case.problem, sf_layout=layout)
    dev = pl.to_device(case.arrays, sf_layout=layout, k=p["k"])
    keep = None
    if discrete:
        empty = [g for g in range(p["num_groups"]) if case.counts[g] == 0]
        ptrs, keep = pl.discrete_weights(p, case.arrays, seed=case.seed, null_empty=empty, sf_layout=layout)
        tensors = pl.inputs_for(p, dev, discrete=ptrs)
    else:
        tensors = pl.inputs_for(p, dev)
    outs = pl.empty_outputs(p, fill=0xA5)
    prev = mg.moegg_set_grid_limit(grid)
    try:
        mg.run(p, {**tensors, **outs})
        torch.cuda.synchronize()
    finally:
        mg.moegg_set_grid_limit(prev)
    del keep
    stats = check_case(case, pl.to_host(outs))
    print(f"[gpu-case] {name} stats {stats}", flush=True)
