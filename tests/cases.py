"""Seeded problem recipes shared by the GPU parity tests and the CPU
cross-check of the two oracles: (base workload, overrides) per case name.
The GPU tests seed case `name` of SMALL with 1000 + its index in sorted(SMALL)
and of EDGE with 2000 + its index in sorted(EDGE)."""

# small cases: every output element against the oracle
SMALL = {
    "gating_l4_full": ("quant_gating_l4", {}),
    "swiglu_fp8_e4m3": ("fc1_swiglu_l8", dict(L=3, K=512, N=320, routing=("topk", 300, 2))),
    "swiglu_fp8_bf16": ("fc1_swiglu_l8", dict(L=3, K=512, N=320, routing=("topk", 300, 2), d="bf16",
                                              alpha=("uniform", 0.5, 2.0))),
    "swiglu_fp8_nc3": ("fc1_swiglu_l8", dict(L=2, K=256, N=256, routing=("topk", 200, 2), norm_const=3.0)),
    "swiglu_fp4_e4m3_c": ("fc1_swiglu_l8", dict(L=2, ab="e2m1x2", K=512, N=320, routing=("topk", 160, 2),
                                                b_std=1.0, clip=6.0, c="bf16")),
    "fc2_zipf_bf16": ("fc2_gating_l64_zipf", dict(L=9, K=384, N=320, routing=("topk_zipf", 400, 3, 1.1, 2))),
    "gating_fp8_e4m3": ("quant_gating_l4", dict(L=3, K=256, N=288, d="e4m3", routing=("multinomial", 300))),
    "srelu_fp4_tanh_e4m3": ("srelu_tanh_fp4_l32", dict(L=3, K=1024, N=320, routing=("multinomial", 500))),
    "srelu_fp4_plain_bf16": ("srelu_tanh_fp4_l32", dict(L=3, K=512, N=256, routing=("multinomial", 300),
                                                        s=0.0, d="bf16", c=None)),
    "srelu_fp8_tanh_bf16_c": ("srelu_tanh_fp4_l32", dict(ab="e4m3", L=2, K=512, N=256, clip=None, s=8.0,
                                                         routing=("multinomial", 300), d="bf16", c="bf16",
                                                         b_std="1/sqrtK")),
    "gating_bf16_ops": ("quant_gating_l4", dict(ab="bf16", K=256, N=320, a_std=1.0, b_std=0.1)),
    "swiglu_bf16_ops_e4m3": ("fc1_swiglu_l8", dict(ab="bf16", L=2, K=192, N=256, routing=("topk", 200, 2))),
    "dswiglu_bf16": ("dswiglu_bf16_l64", dict(L=5, K=256, N=288, routing=("topk", 200, 3),
                                              alpha=("uniform", 0.5, 2.0), beta=("uniform", 0.5, 2.0))),
    # block-scaled dSwiGLU ("Grouped GEMM + dGLU (SM100)", block-scaled contract):
    # step counts 8 (even), 5 (odd), 3 and 2 exercise every load schedule
    "dswiglu_mxfp8_e4m3": ("dswiglu_mxfp8_l64", dict(L=5, K=1024, N=288, routing=("topk", 200, 3),
                                                     alpha=("uniform", 0.5, 2.0), beta=("uniform", 0.5, 2.0))),
    "dswiglu_mxfp8_e4m3_odd": ("dswiglu_mxfp8_l64", dict(L=3, K=640, N=256, routing=("topk", 150, 2),
                                                         norm_const=2.0)),
    "dswiglu_mxfp8_bf16_amax": ("dswiglu_mxfp8_l64", dict(L=4, K=384, N=320, d="bf16", routing=("topk", 200, 2),
                                                          alpha=("uniform", 0.5, 2.0))),
    "dswiglu_mxfp4_e4m3": ("dswiglu_mxfp8_l64", dict(ab="e2m1x2", L=3, K=512, N=256, routing=("topk", 150, 2),
                                                     a_std=1.0, b_std=1.0, clip=6.0)),
    "dswiglu_mxfp4_bf16_amax": ("dswiglu_mxfp8_l64", dict(ab="e2m1x2", d="bf16", L=3, K=1024, N=288,
                                                          routing=("topk", 150, 2), a_std=1.0, b_std=1.0,
                                                          clip=6.0)),
    # sReLU backward (tanh clamp s = 8 and plain s = 0), every operand family
    "dsrelu_mxfp8_e4m3": ("dsrelu_mxfp8_l32", dict(L=3, K=1024, N=320, routing=("multinomial", 300),
                                                   alpha=("uniform", 0.5, 2.0))),
    "dsrelu_mxfp8_e4m3_odd_plain": ("dsrelu_mxfp8_l32", dict(L=2, K=640, N=256, routing=("multinomial", 200),
                                                             s=0.0, norm_const=0.5)),
    "dsrelu_mxfp4_bf16_amax": ("dsrelu_mxfp8_l32", dict(ab="e2m1x2", d="bf16", L=3, K=1024, N=288,
                                                        routing=("multinomial", 300), a_std=1.0, b_std=1.0,
                                                        clip=6.0)),
    "dsrelu_bf16_ops": ("dsrelu_mxfp8_l32", dict(ab="bf16", d="bf16", L=2, K=192, N=256,
                                                 routing=("multinomial", 200))),
    # E2M1 operands with FP8 dC and a last wave column holding one 32-column
    # block (N % 64 == 32): the C_in staging's half-empty row
    "dsrelu_mxfp4_e4m3_n288": ("dsrelu_mxfp8_l32", dict(ab="e2m1x2", L=3, K=512, N=288,
                                                        routing=("multinomial", 300), a_std=1.0, b_std=1.0,
                                                        clip=6.0)),
    # E5M2 operands ("Grouped GEMM + Quant", §Data Types) through the other epilogues
    "e5m2_gating_bf16": ("quant_gating_l4", dict(ab="e5m2", L=3, K=384, N=288, routing=("multinomial", 300))),
    "e5m2_swiglu_e4m3": ("fc1_swiglu_l8", dict(ab="e5m2", L=3, K=640, N=320, routing=("topk", 300, 2))),
    # GeGLU forward: clamps that bite (|C| ~ 1 against bounds -1.5 / 1), other
    # constants, every operand family, both output formats
    "geglu_e5m2_e4m3_clamped": ("fc1_geglu_e5m2_l8", dict(L=3, K=1024, N=320, routing=("topk", 300, 2),
                                                          glu_clamp_min=-1.5, glu_clamp_max=1.0)),
    "geglu_fp8_bf16_consts": ("fc1_geglu_e5m2_l8", dict(ab="e4m3", d="bf16", L=3, K=384, N=256,
                                                        routing=("topk", 200, 2), glu_gamma=0.75,
                                                        geglu_alpha=1.25, linear_offset=0.5,
                                                        glu_clamp_min=float("-inf"), glu_clamp_max=float("inf"),
                                                        alpha=("uniform", 0.5, 2.0))),
    "geglu_fp4_e4m3_c": ("fc1_geglu_e5m2_l8", dict(ab="e2m1x2", L=2, K=512, N=320, routing=("topk", 160, 2),
                                                   b_std=1.0, clip=6.0, c="bf16", glu_clamp_min=-4.0,
                                                   glu_clamp_max=3.0)),
    "geglu_bf16_ops": ("fc1_geglu_e5m2_l8", dict(ab="bf16", L=2, K=192, N=256, routing=("topk", 200, 2),
                                                 glu_clamp_min=-0.75, glu_clamp_max=0.75)),
    # dGeGLU backward ("Grouped GEMM + dGLU (SM100)", dGeGLU): C ~ N(0, 4^2)
    # against clamps -7 / 7, so both masks and the sigmoid tails are exercised
    "dgeglu_mxfp8_e4m3": ("dgeglu_mxfp8_l64", dict(L=5, K=1024, N=288, routing=("topk", 200, 3),
                                                   alpha=("uniform", 0.5, 2.0))),
    "dgeglu_e5m2_bf16_amax": ("dgeglu_mxfp8_l64", dict(ab="e5m2", d="bf16", L=3, K=640, N=256,
                                                       routing=("topk", 150, 2), linear_offset=0.25,
                                                       glu_clamp_min=-3.0, glu_clamp_max=5.0)),
    "dgeglu_mxfp4_e4m3": ("dgeglu_mxfp8_l64", dict(ab="e2m1x2", L=3, K=512, N=256, routing=("topk", 150, 2),
                                                   a_std=1.0, b_std=1.0, clip=6.0, norm_const=2.0)),
    "dgeglu_bf16_ops": ("dgeglu_mxfp8_l64", dict(ab="bf16", d="bf16", L=2, K=192, N=288,
                                                 routing=("topk", 150, 2), geglu_alpha=1.0)),
    "dgeglu_mxfp4_bf16_amax_n288": ("dgeglu_mxfp8_l64", dict(ab="e2m1x2", d="bf16", L=3, K=512, N=288,
                                                             routing=("topk", 150, 2), a_std=1.0, b_std=1.0,
                                                             clip=6.0)),
}

# edge cases
EDGE = {
    # empty first / middle / last groups, single-row groups, a group of exactly 128
    "edge_groups_gating": ("quant_gating_l4", dict(L=7, K=256, N=256, force_counts=[0, 1, 0, 128, 129, 0, 1])),
    "edge_groups_swiglu_e4m3": ("fc1_swiglu_l8", dict(L=5, K=128, N=128, force_counts=[0, 1, 200, 0, 3])),
    "edge_l1": ("quant_gating_l4", dict(L=1, K=128, N=64, force_counts=[5])),
    "edge_n64_swiglu": ("fc1_swiglu_l8", dict(L=2, K=128, N=64, routing=("topk", 100, 1))),
    "edge_k_one_step_fp4": ("srelu_tanh_fp4_l32", dict(L=2, K=256, N=64, routing=("multinomial", 70))),
    "edge_k_one_step_bf16": ("dswiglu_bf16_l64", dict(L=2, K=64, N=32, routing=("topk", 50, 1))),
    # the maximum expert count: 1024 groups, most of them empty, the first and
    # the last one populated (the whole tile prefix and its search)
    "edge_l1024_sparse": ("quant_gating_l4", dict(L=1024, K=128, N=64,
                                                  force_counts=[3] + [0] * 200 + [130] + [0] * 300 + [1]
                                                  + [0] * 400 + [257] + [0] * 119 + [2])),
    # groups aligned to 256 rows (the pages' default padding)
    "edge_m_aligned_256": ("fc1_swiglu_l8", dict(L=3, K=256, N=128, m_aligned=256, routing=("topk", 300, 2))),
}

# SwiGLU over E2M1 operands with E4M3 D where a column block holds one
# routed row whose gates lie near -88: the sigmoid of those gates is below
# FP32's normal range, so the FP32 epilogue gives 0 where the float64 oracle
# keeps ~1e-35 (drawn by a randomized run; seed of each case given here)
UNDERFLOW = {
    "underflow_swiglu_fp4_l26_zipf": ("fc1_swiglu_l8", dict(
        ab="e2m1x2", d="e4m3", c=None, L=26, K=2816, N=1024, m_aligned=128, alpha=("uniform", 0.5, 2.0),
        routing=("topk_zipf", 5721, 3, 1.1, 2), prob=("softmax_picks",), a_std=1.0, b_std=1.0, clip=6.0), 20163),
    "underflow_swiglu_fp4_l59": ("fc1_swiglu_l8", dict(
        ab="e2m1x2", d="e4m3", c=None, L=59, K=1024, N=640, m_aligned=256, alpha=("uniform", 0.5, 2.0),
        routing=("multinomial", 5355), prob=("uniform",), a_std=1.0, b_std=1.0, clip=6.0), 20164),
    "underflow_swiglu_fp4_l22_c_nc4": ("fc1_swiglu_l8", dict(
        ab="e2m1x2", d="e4m3", c="bf16", L=22, K=1792, N=1216, m_aligned=128, alpha=("uniform", 0.5, 2.0),
        routing=("multinomial", 5751), prob=("uniform",), a_std=1.0, b_std=1.0, clip=6.0, norm_const=4.0), 20242),
}

# sReLU backward deep in the tanh clamp (s = 0.5 against C_in ~ N(0, 4^2), so
# relu(C)/s reaches ~30): the gradient's factor 1 - tanh^2 = sech^2 must be
# evaluated without the cancellation of 1 - t*t, on both sides (drawn by
# randomized runs; seed of each case given here)
SATURATED = {
    "saturated_dsrelu_fp8_l48_n352": ("dsrelu_mxfp8_l32", dict(
        ab="e4m3", d="e4m3", c=None, L=48, K=256, N=352, m_aligned=128, alpha=("uniform", 0.5, 2.0),
        routing=("multinomial", 5537), prob=("uniform",), s=0.5), 20041),
    "saturated_dsrelu_fp4_l51_zipf": ("dsrelu_mxfp8_l32", dict(
        ab="e2m1x2", d="e4m3", c=None, L=51, K=768, N=480, m_aligned=256, alpha=("uniform", 0.5, 2.0),
        routing=("topk_zipf", 3197, 3, 1.1, 2), prob=("softmax_picks",), a_std=1.0, b_std=1.0, clip=6.0,
        s=0.5), 20213),
    "saturated_dsrelu_fp8_l24_bf16dc": ("dsrelu_mxfp8_l32", dict(
        ab="e4m3", d="bf16", c=None, L=24, K=1152, N=384, m_aligned=256, alpha=("uniform", 0.5, 2.0),
        routing=("topk", 3188, 2), prob=("softmax_picks",), s=0.5), 20261),
}

# value ranges far from the workloads' (alpha 1e2..1e3 or 1e-3..1e-2, operand
# spreads up to 20): C is large with heavy cancellation, and where it lands in
# the narrow range in which a saturating activation (GeGLU's clamps, sReLU's
# tanh clamp) still moves, or where R is smaller than its own accumulation
# error, the FP32 / matrix-core accumulation error moves D beyond 1e-2 of the
# group's largest output or a block's scale byte by more than one binade;
# parity then rests on the outputs' accumulation envelopes (drawn by
# randomized runs; seed of each case given here)
EXTREME = {
    "extreme_srelu_tanh_fp8_alpha1e3": ("srelu_tanh_fp4_l32", dict(
        ab="e4m3", d="bf16", c=None, L=41, K=256, N=32, m_aligned=256, alpha=("uniform", 100.0, 1000.0),
        routing=("multinomial", 611), prob=("uniform",), s=8.0, a_std=20.0, b_std=1.0), 20211),
    "extreme_geglu_fp8_alpha1e3": ("fc1_geglu_e5m2_l8", dict(
        ab="e4m3", d="bf16", c=None, L=3, K=1024, N=1024, m_aligned=128, alpha=("uniform", 100.0, 1000.0),
        routing=("topk", 1988, 2), prob=("softmax_picks",), glu_clamp_min=-4.372481653726602,
        glu_clamp_max=3.9092775713363848, a_std=1.0, b_std=1.0, glu_gamma=1.8713954712937324,
        geglu_alpha=2.741583703283421, linear_offset=1.7249855711340354), 20134),
    "extreme_geglu_e5m2_wide_operands": ("fc1_geglu_e5m2_l8", dict(
        ab="e5m2", d="bf16", c="bf16", L=10, K=1152, N=768, m_aligned=256, alpha=("uniform", 100.0, 1000.0),
        routing=("topk_zipf", 1342, 3, 1.1, 2), prob=("softmax_picks",), glu_clamp_min=-1.2312725358369347,
        glu_clamp_max=5.75180580090614, norm_const=4.0, a_std=20.0, b_std=10.0, glu_gamma=1.1420180543826177,
        geglu_alpha=1.7548918880311337, linear_offset=1.6171785910121055), 20215),
    "extreme_dgeglu_fp8_alpha1e-3": ("dgeglu_mxfp8_l64", dict(
        ab="e4m3", d="e4m3", c=None, L=20, K=512, N=448, m_aligned=128, alpha=("uniform", 0.001, 0.01),
        routing=("topk_zipf", 1575, 3, 1.1, 2), prob=("softmax_picks",), glu_clamp_min=-3.936643832437433,
        glu_clamp_max=6.536454994200406, a_std=0.1, b_std=10.0, c_std=40.0, glu_gamma=0.27401165755352885,
        geglu_alpha=2.463042990743805, linear_offset=-0.17798175842376684), 20211),
}
