"""The persistent tile loop's tile-to-tile hand-offs, every output against the
oracle.

Each workgroup of the kernel walks a list of output tiles; between two tiles
it loads the next tile's first stage (during the last two K-steps for an even
step count >= 4, else during the epilogue) and reuses its LDS scratch and
staged prob.  A problem small enough for the oracle has fewer tiles than the
GPU has compute units, so these cases cap the grid at 1-3 workgroups with the
library's testing hook (moegg_set_grid_limit): every workgroup then runs many
tiles in a row.  The step counts 1-8 cover every load schedule (1-2, 3, odd
>= 5, even >= 4 steps per tile).  Five larger cases (> 512 tiles) run at the
natural grid of one workgroup per compute unit, where each workgroup takes
two or three tiles, including a last pass with 3 and with 255 tiles left.
("Grouped GEMM + Quant (SM100)", §Equations, Step 1:
rows are grouped over every expert range, whichever workgroup computes
them.)"""
import pytest

import synth
from test_gpu_parity import check_case, run_gpu

pytestmark = pytest.mark.gpu

mg = pytest.importorskip("moe_grouped_block_amd")

SW = dict(routing=("topk", 800, 2))          # 3 experts, 1600 routed rows: ~7 row tiles
CASES = {
    # 8-bit operands, K-steps = K / 128
    "pers_swiglu_e4m3_k1_g1": ("fc1_swiglu_l8", dict(L=3, K=128, N=320, **SW), 1),
    "pers_swiglu_e4m3_k2_g2": ("fc1_swiglu_l8", dict(L=3, K=256, N=320, **SW), 2),
    "pers_swiglu_e4m3_k3_g1": ("fc1_swiglu_l8", dict(L=3, K=384, N=320, **SW), 1),
    "pers_swiglu_e4m3_k4_g3": ("fc1_swiglu_l8", dict(L=3, K=512, N=320, **SW), 3),
    "pers_swiglu_e4m3_k5_g2": ("fc1_swiglu_l8", dict(L=3, K=640, N=320, **SW), 2),
    "pers_swiglu_e4m3_k6_g1": ("fc1_swiglu_l8", dict(L=3, K=768, N=320, **SW), 1),
    "pers_swiglu_e4m3_k8_g2": ("fc1_swiglu_l8", dict(L=3, K=1024, N=320, **SW), 2),
    "pers_gating_bf16_k1_g1": ("quant_gating_l4", dict(L=4, K=128, N=288, routing=("multinomial", 1800)), 1),
    "pers_gating_bf16_k3_g2": ("quant_gating_l4", dict(L=4, K=384, N=288, routing=("multinomial", 1800),
                                                       c="bf16"), 2),
    "pers_gating_bf16_k4_g1": ("quant_gating_l4", dict(L=4, K=512, N=288, routing=("multinomial", 1800)), 1),
    "pers_gating_bf16_k7_g3": ("quant_gating_l4", dict(L=4, K=896, N=288, routing=("multinomial", 1800)), 3),
    # backward activations: FP8 dC (staged C_in, column scales), BF16 dC + amax (L, 2)
    "pers_dswiglu_e4m3_k2_g1": ("dswiglu_mxfp8_l64", dict(L=3, K=256, N=288, routing=("topk", 800, 2),
                                                          alpha=("uniform", 0.5, 2.0),
                                                          beta=("uniform", 0.5, 2.0)), 1),
    "pers_dswiglu_e4m3_k4_g2": ("dswiglu_mxfp8_l64", dict(L=3, K=512, N=288, routing=("topk", 800, 2)), 2),
    "pers_dswiglu_e4m3_k5_g1": ("dswiglu_mxfp8_l64", dict(L=3, K=640, N=256, routing=("topk", 800, 2)), 1),
    "pers_dswiglu_bf16amax_k3_g2": ("dswiglu_mxfp8_l64", dict(L=3, K=384, N=320, d="bf16",
                                                              routing=("topk", 800, 2)), 2),
    "pers_dsrelu_e4m3_k6_g1": ("dsrelu_mxfp8_l32", dict(L=3, K=768, N=320, routing=("multinomial", 1800)), 1),
    "pers_dgeglu_e4m3_k3_g3": ("dgeglu_mxfp8_l64", dict(L=3, K=384, N=256, routing=("topk", 800, 2)), 3),
    # BF16 operands (K-steps = K / 64) and E2M1 operands (K-steps = K / 256)
    "pers_dswiglu_bf16ops_k2_g1": ("dswiglu_bf16_l64", dict(L=3, K=128, N=288, routing=("topk", 800, 2)), 1),
    "pers_dswiglu_bf16ops_k5_g2": ("dswiglu_bf16_l64", dict(L=3, K=320, N=256, routing=("topk", 800, 2)), 2),
    "pers_srelu_fp4_e4m3_k1_g1": ("srelu_tanh_fp4_l32", dict(L=3, K=256, N=320, routing=("multinomial", 1800)), 1),
    "pers_srelu_fp4_e4m3_c_k4_g2": ("srelu_tanh_fp4_l32", dict(L=3, K=1024, N=320, routing=("multinomial", 1800),
                                                               c="bf16"), 2),
    "pers_srelu_fp4_e4m3_k3_g3": ("srelu_tanh_fp4_l32", dict(L=3, K=768, N=256, routing=("multinomial", 1800)), 3),
}


@pytest.mark.parametrize("name", list(CASES))
def test_persistent_multi_tile(name):
    base, over, grid = CASES[name]
    case = synth.make_case(base, seed=6000 + sorted(CASES).index(name), name=name, **over)
    print(f"[gpu-case] {name} grid limit {grid}", flush=True)
    prev = mg.moegg_set_grid_limit(grid)
    try:
        got = run_gpu(case)
    finally:
        mg.moegg_set_grid_limit(prev)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)


# more than 512 tiles of 256 x 256 at the natural grid (one workgroup per CU)
BIG = {
    "big_gating_bf16_k5": ("quant_gating_l4", dict(L=4, K=640, N=512, routing=("multinomial", 70000))),
    "big_swiglu_e4m3_k4": ("fc1_swiglu_l8", dict(L=4, K=512, N=512, routing=("multinomial", 70000),
                                                 prob=("uniform",))),
    "big_dswiglu_e4m3_k3": ("dswiglu_mxfp8_l64", dict(L=4, K=384, N=512, routing=("multinomial", 70000),
                                                      prob=("uniform",))),
    # the last, partial pass is dealt evenly over the 8 XCDs: 515 tiles leave
    # 3 for it (most XCDs get none), 767 tiles leave 255
    "big_gating_rem3": ("quant_gating_l4", dict(L=1, K=128, N=256, force_counts=[515 * 256])),
    "big_gating_rem255": ("quant_gating_l4", dict(L=1, K=128, N=256, force_counts=[767 * 256], d="e4m3")),
}


@pytest.mark.parametrize("name", list(BIG))
def test_many_tiles_natural_grid(name):
    base, over = BIG[name]
    case = synth.make_case(base, seed=6500 + sorted(BIG).index(name), name=name, **over)
    vm, n = case.problem["valid_m"], case.problem["n"]
    assert (vm // 256) * ((n + 255) // 256) > 512
    got = run_gpu(case)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)
