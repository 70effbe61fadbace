"""The two scale layouts of the C ABI on the GPU.

* moegg_sf_to_kplanes against the plane formula: byte kb of row r of a
  row-major (rows, K/32) array lands at 4 * ((kb // 4) * rows + r) + kb % 4.
* sf_layout = KPLANES through the kernel: the same logical scales laid out
  as planes give every output bit for bit as the row-major layout does (the
  kernel reads the same bytes), and match the oracle.
("Grouped GEMM + Quant (SM100)", §Shapes: one E8M0 byte per 32 K elements of
every row of A and B; the plane layout is this library's.)"""
import numpy as np
import pytest

import synth
from test_gpu_parity import _announce, assert_same_as_dense, check_case, run_gpu

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mg = pytest.importorskip("moe_grouped_block_amd")
from moe_grouped_block_amd import plumbing as pl  # noqa: E402


@pytest.mark.parametrize("rows,k", [(1000, 640), (1, 128), (4097, 256), (129, 4096)])
def test_sf_to_kplanes_matches_formula(rows, k):
    print(f"\n[gpu-case] sf_to_kplanes rows={rows} k={k}", flush=True)
    rng = np.random.default_rng(rows + k)
    logical = rng.integers(0, 256, (rows, k // 32), dtype=np.uint8)
    src = torch.from_numpy(logical).cuda()
    dst = torch.full((rows * k // 32,), 0xA5, dtype=torch.uint8, device="cuda")
    mg.sf_to_kplanes(src, dst, rows, k)
    torch.cuda.synchronize()
    got = dst.cpu().numpy()
    r = np.arange(rows)[:, None]
    kb = np.arange(k // 32)[None, :]
    expect = np.empty_like(got)
    expect[4 * ((kb // 4) * rows + r) + kb % 4] = logical
    assert np.array_equal(got, expect)


def run_gpu_kplanes(case, fill=0xA5, discrete=False):
    """Run with the scales laid out as K-block planes on the device."""
    _announce(case)
    print(f"[gpu-case] {case.name} sf_layout kplanes{' discrete' if discrete else ''}", flush=True)
    p = dict(case.problem, sf_layout="kplanes")
    dev = pl.to_device(case.arrays, sf_layout="kplanes", k=p["k"])
    keep = None
    if discrete:
        ptrs, keep = pl.discrete_weights(p, case.arrays, seed=case.seed, sf_layout="kplanes")
        tensors = pl.inputs_for(p, dev, discrete=ptrs)
    else:
        tensors = pl.inputs_for(p, dev)
    outs = pl.empty_outputs(p, fill=fill)
    mg.run(p, {**tensors, **outs})
    torch.cuda.synchronize()
    del keep
    return pl.to_host(outs)


CASES = {
    "kplanes_swiglu_fp8_e4m3": ("fc1_swiglu_l8", dict(L=3, K=512, N=320, routing=("topk", 300, 2)), False, 0),
    "kplanes_srelu_fp4_e4m3_c": ("srelu_tanh_fp4_l32", dict(L=3, K=1024, N=320, routing=("multinomial", 500),
                                                            c="bf16"), False, 0),
    "kplanes_dswiglu_e4m3_odd": ("dswiglu_mxfp8_l64", dict(L=3, K=640, N=256, routing=("topk", 150, 2)), False, 0),
    "kplanes_gating_discrete_empty": ("quant_gating_l4", dict(L=7, K=512, N=256,
                                                              force_counts=[0, 1, 0, 128, 129, 0, 1]), True, 0),
    "kplanes_geglu_e5m2_grid2": ("fc1_geglu_e5m2_l8", dict(L=3, K=768, N=320, routing=("topk", 800, 2)), False, 2),
}


@pytest.mark.parametrize("name", list(CASES))
def test_kplanes_parity(name):
    base, over, discrete, grid = CASES[name]
    case = synth.make_case(base, seed=7000 + sorted(CASES).index(name), name=name, **over)
    prev = mg.moegg_set_grid_limit(grid)
    try:
        got = run_gpu_kplanes(case, discrete=discrete)
        ref_rows = run_gpu(case)
    finally:
        mg.moegg_set_grid_limit(prev)
    assert_same_as_dense(got, ref_rows)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)
