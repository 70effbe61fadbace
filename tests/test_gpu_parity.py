"""GPU parity: the HIP library (through the C ABI) against the oracle.

Small cases run the oracle on every output; full-size workloads compare
sampled whole 32-row blocks plus properties that hold at any size.  Every case
prints its name, seed and shape before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import formats as F
from cases import EDGE, EXTREME, SATURATED, SMALL, UNDERFLOW
import parity_util
from parity_util import (acc_error_bound, amax_rule, decode_bf16, make_envelope, make_refine, pick_row_blocks,
                         row_col_consistency, rule1, rule2, underflow_mask)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
mg = pytest.importorskip("moe_grouped_block_amd")
from moe_grouped_block_amd import plumbing as pl  # noqa: E402


def _announce(case):
    p = case.problem
    print(f"\n[gpu-case] {case.name} seed={case.seed} L={p['num_groups']} valid_m={p['valid_m']} "
          f"n={p['n']} k={p['k']} ab={p['ab_dtype']} act={p['act']} d={p['d_dtype']} c={p.get('c_dtype')}",
          flush=True)


def run_gpu(case, fill=0xA5, times=1):
    _announce(case)
    dev = pl.to_device(case.arrays)
    res = []
    for _ in range(times):
        outs = pl.empty_outputs(case.problem, fill=fill)
        mg.run(case.problem, {**pl.inputs_for(case.problem, dev), **outs})
        torch.cuda.synchronize()
        res.append(pl.to_host(outs))
    return res if times > 1 else res[0]


def check_case(case, got, rows=None):
    """Compare GPU outputs with the oracle on `rows` (default all rows)."""
    p = case.problem
    ref = oracle.grouped_gemm(p, case.arrays, rows)
    r = ref["rows"]
    grp = ref["group"]
    stats = {}
    if p["act"] in ("dswiglu", "dsrelu", "dgeglu"):
        stats["dprob"] = rule1(got["dprob"][r], ref["dprob"], grp, "dprob")
        if p["d_dtype"] == "e4m3":
            nc = float(case.arrays["norm_const"][0])
            rb = acc_error_bound(case, ref)
            fz = underflow_mask(case, ref)
            stats["d_row"] = rule2(got["d"][r], got["sfd_row"][r], ref["dc"], nc, "row", "dC/SFD_row", rb,
                                   make_refine(case, ref, "row"), fz)
            blocks = np.unique(r // 32)
            stats["d_col"] = rule2(got["d_col"][r], got["sfd_col"][:, blocks], ref["dc"], nc, "col",
                                   "dC_col/SFD_col", rb, make_refine(case, ref, "col"), fz)
            return stats
        g2 = np.repeat(grp[:, None], ref["dc"].shape[1], axis=1)
        stats["dc"] = rule1(decode_bf16(got["d"][r]), ref["dc"], g2, "dC", make_envelope(case, ref))
        if "amax2" in ref and rows is None:
            stats["amax2"] = amax_rule(got["amax"].reshape(-1), ref["amax2"].reshape(-1))
        if "amax" in ref and rows is None:
            stats["amax"] = amax_rule(got["amax"], ref["amax"])
        return stats
    if p.get("c_dtype") == "bf16":
        g2 = np.repeat(grp[:, None], ref["c"].shape[1], axis=1)
        stats["c"] = rule1(decode_bf16(got["c"][r]), ref["c"], g2, "C")
    if p["d_dtype"] == "bf16":
        g2 = np.repeat(grp[:, None], ref["d"].shape[1], axis=1)
        stats["d"] = rule1(decode_bf16(got["d"][r]), ref["d"], g2, "D", make_envelope(case, ref))
        if rows is None:
            stats["amax"] = amax_rule(got["amax"], ref["amax"])
    else:
        nc = float(case.arrays["norm_const"][0])
        rb = acc_error_bound(case, ref)
        fz = underflow_mask(case, ref)
        stats["d_row"] = rule2(got["d"][r], got["sfd_row"][r], ref["d"], nc, "row", "D/SFD_row", rb,
                               make_refine(case, ref, "row"), fz)
        blocks = np.unique(r // 32)
        stats["d_col"] = rule2(got["d_col"][r], got["sfd_col"][:, blocks], ref["d"], nc, "col", "D_col/SFD_col", rb,
                               make_refine(case, ref, "col"), fz)
    return stats


# ---------------------------------------------------------------------------
# small cases: every output element against the oracle
# ---------------------------------------------------------------------------

# SMALL: see tests/cases.py


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(name):
    base, over = SMALL[name]
    case = synth.make_case(base, seed=1000 + sorted(SMALL).index(name), name=name, **over)
    got = run_gpu(case)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)


# The epilogue stores each 32-row block of a wave's outputs in whole row
# segments of its 64 GEMM columns.  With N = 32 mod 64 the last wave has one
# 32-column block only and must store half of each segment: the C store (and
# D) of the forward sReLU, whose other paths have such a case above.
# ("Grouped GEMM + sReLU (SM100)", §Equations: C and D cover columns [0, N).)
HALF_SEGMENT = {
    "half_segment_srelu_fp8_c_e4m3": ("srelu_tanh_fp4_l32", dict(ab="e4m3", L=3, K=512, N=288, clip=None, s=8.0,
                                                                 routing=("multinomial", 400), c="bf16",
                                                                 b_std="1/sqrtK")),
    "half_segment_srelu_fp4_c_bf16": ("srelu_tanh_fp4_l32", dict(L=2, K=512, N=288, routing=("multinomial", 300),
                                                                 c="bf16", d="bf16")),
}


@pytest.mark.parametrize("name", list(HALF_SEGMENT))
def test_half_segment_parity(name):
    base, over = HALF_SEGMENT[name]
    case = synth.make_case(base, seed=1500 + sorted(HALF_SEGMENT).index(name), name=name, **over)
    got = run_gpu(case)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

# EDGE: see tests/cases.py


@pytest.mark.parametrize("name", list(SATURATED))
def test_saturated_tanh_clamp_backward_parity(name):
    """dsReLU with s = 0.5: most gradients sit deep in the tanh clamp, where
    1 - tanh^2 must be evaluated as sech^2 (no cancellation) to match."""
    base, over, seed = SATURATED[name]
    case = synth.make_case(base, seed=seed, name=name, **over)
    got = run_gpu(case)
    stats = check_case(case, got)
    print(f"[gpu-case] {name} stats {stats}", flush=True)


@pytest.mark.parametrize("name", list(UNDERFLOW))
def test_fp32_underflow_parity(name):
    """Blocks carried by sigmoid factors below FP32's normal range: the
    library's FP32 epilogue gives 0 there; parity holds with those elements
    at 0 (rule 2's `fragile`), and the case does reach that path."""
    base, over, seed = UNDERFLOW[name]
    case = synth.make_case(base, seed=seed, name=name, **over)
    got = run_gpu(case)
    stats = check_case(case, got)
    assert stats["d_col"]["scale_fp32_underflow"] > 0
    print(f"[gpu-case] {name} stats {stats}", flush=True)


@pytest.mark.parametrize("name", list(EXTREME))
def test_extreme_range_parity(name):
    """C large with heavy cancellation under saturating activations, or R
    below its own accumulation error: parity holds with the outputs'
    accumulation envelopes, and the case does reach them."""
    base, over, seed = EXTREME[name]
    case = synth.make_case(base, seed=seed, name=name, **over)
    got = run_gpu(case)
    n0 = len(parity_util.RULE1_LOG)
    stats = check_case(case, got)
    enveloped = sum(a for _, a, _ in parity_util.RULE1_LOG[n0:])
    enveloped += sum(v.get("scale_mfma_truncation", 0) for v in stats.values() if isinstance(v, dict))
    assert enveloped > 0
    print(f"[gpu-case] {name} stats {stats} enveloped {enveloped}", flush=True)


@pytest.mark.parametrize("name", list(EDGE))
def test_edge_parity(name):
    base, over = EDGE[name]
    case = synth.make_case(base, seed=2000 + sorted(EDGE).index(name), name=name, **over)
    got = run_gpu(case)
    check_case(case, got)


# ---------------------------------------------------------------------------
# discrete weights: the same logical B through per-expert allocations
# ("Grouped GEMM + sReLU (SM100)", §Discrete-weight wrapper; b_ptrs/sfb_ptrs)
# ---------------------------------------------------------------------------

DISCRETE = {
    "discrete_swiglu_fp8_e4m3": ("fc1_swiglu_l8", dict(L=3, K=512, N=320, routing=("topk", 300, 2))),
    "discrete_srelu_fp4_e4m3_c": ("srelu_tanh_fp4_l32", dict(L=3, K=512, N=320, routing=("multinomial", 300),
                                                             c="bf16")),
    "discrete_fc2_odd_steps_bf16": ("fc2_gating_l64_zipf", dict(L=9, K=384, N=320,
                                                                routing=("topk_zipf", 400, 3, 1.1, 2))),
    "discrete_dswiglu_bf16": ("dswiglu_bf16_l64", dict(L=4, K=256, N=288, routing=("topk", 200, 3))),
    "discrete_empty_groups": ("quant_gating_l4", dict(L=7, K=512, N=256, force_counts=[0, 1, 0, 128, 129, 0, 1])),
    "discrete_dgeglu_e5m2_e4m3": ("dgeglu_mxfp8_l64", dict(ab="e5m2", L=4, K=512, N=256, routing=("topk", 200, 3))),
}


def run_gpu_discrete(case, fill=0xA5):
    """Run with per-expert weight allocations; experts without rows get null
    pointers (the library never reads them)."""
    _announce(case)
    print(f"[gpu-case] {case.name} discrete weights", flush=True)
    dev = pl.to_device(case.arrays)
    empty = [g for g in range(case.problem["num_groups"]) if case.counts[g] == 0]
    ptrs, keep = pl.discrete_weights(case.problem, case.arrays, seed=case.seed, null_empty=empty)
    outs = pl.empty_outputs(case.problem, fill=fill)
    mg.run(case.problem, {**pl.inputs_for(case.problem, dev, discrete=ptrs), **outs})
    torch.cuda.synchronize()
    del keep
    return pl.to_host(outs)


def assert_same_as_dense(got, dense):
    for k in got:
        if k == "dprob":        # accumulated with atomics: the order varies between runs
            continue
        assert np.array_equal(got[k], dense[k]), f"{k} differs between discrete and dense weights"


@pytest.mark.parametrize("name", list(DISCRETE))
def test_discrete_weights_parity(name):
    base, over = DISCRETE[name]
    case = synth.make_case(base, seed=4000 + sorted(DISCRETE).index(name), name=name, **over)
    got = run_gpu_discrete(case)
    stats = check_case(case, got)
    assert_same_as_dense(got, run_gpu(case))
    print(f"[gpu-case] {name} stats {stats}", flush=True)


def test_empty_problem_fills_amax():
    case = synth.make_case("quant_gating_l4", seed=3, name="all_empty", L=3, force_counts=[0, 0, 0])
    assert case.problem["valid_m"] == 0
    _announce(case)
    dev = pl.to_device({k: v for k, v in case.arrays.items() if v.size})
    amax = torch.full((3,), 7.0, device="cuda")
    # zero-row A/prob tensors are represented by any aligned device pointer
    dummy = torch.zeros(64, dtype=torch.uint8, device="cuda")
    t = dict(a=dummy, b=dev["b"], sfa=dummy, sfb=dev["sfb"], padded_offsets=dev["padded_offsets"],
             alpha=dev["alpha"], prob=dummy, d=dummy, amax=amax)
    mg.run(case.problem, t)
    torch.cuda.synchronize()
    assert amax.cpu().tolist() == [0.0, 0.0, 0.0]


def test_row_group_map_bit_exact():
    """alpha_g = 2^g with all-ones data: every row's value is 128 * 2^g, exactly."""
    counts = [0, 3, 130, 0, 1, 255, 0]
    L = len(counts)
    case = synth.make_case("quant_gating_l4", seed=4, name="group_map", L=L, K=128, N=256, force_counts=counts)
    a = case.arrays
    valid = case.row_valid
    a["a"][:] = 0
    a["a"][valid] = 0x38
    a["sfa"][:] = 127
    a["b"][:] = 0x38
    a["sfb"][:] = 127
    a["alpha"][:] = (2.0 ** np.arange(L)).astype(np.float32)
    a["prob"][:] = 1.0
    got = run_gpu(case)
    d = decode_bf16(got["d"])
    grp = oracle.group_of_rows(a["padded_offsets"], np.arange(case.problem["valid_m"]))
    expect = np.where(valid, 128.0 * 2.0 ** grp, 0.0)
    assert np.array_equal(d, np.repeat(expect[:, None], 256, axis=1))
    assert got["amax"].tolist() == [128.0 * 2 ** g if counts[g] else 0.0 for g in range(L)]


def test_e4m3_rounding_through_epilogue_bit_exact():
    """D = prob[m] * 2^e(n) exactly (one nonzero product per dot), so the GPU's
    fp32 D equals the oracle's float32 D and every code and scale must match
    bit for bit: this sweeps the conversion's rounding (ties, subnormals)."""
    rows, n, k = 1024, 256, 128
    case = synth.make_case("quant_gating_l4", seed=5, name="e4m3_rounding", L=1, K=k, N=n, d="e4m3",
                           force_counts=[rows])
    a = case.arrays
    a["a"][:] = 0
    a["a"][:, 0] = 0x38                                       # A[m, 0] = 1, rest 0
    a["sfa"][:] = 127
    a["b"][:] = 0
    e = (np.arange(n) % 32) // 2                              # 0..15 per 32-column block
    a["b"][0, :, 0] = 0x38
    a["sfb"][0, :, 0] = (127 - e).astype(np.uint8)            # B[n, 0] = 2^-e(n)
    a["sfb"][0, :, 1:] = 127
    a["alpha"][:] = 1.0
    rng = np.random.default_rng(55)
    prob = rng.uniform(0.5, 1.0, rows).astype(np.float32)
    # rows whose row-block values land exactly on E4M3 rounding ties: with
    # prob = mid * 2^-9 the row scale is a power of two that maps prob onto a
    # midpoint of the top binades
    pos = F.decode_e4m3(np.arange(0x40, 0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2)
    prob[:len(mids)] = (mids * 2.0 ** -9).astype(np.float32)
    a["prob"][:] = prob
    got = run_gpu(case)
    ref = oracle.grouped_gemm(case.problem, a)
    assert np.array_equal(got["sfd_row"], ref["sfd_row"])
    assert np.array_equal(got["d"], ref["d_code"])
    assert np.array_equal(got["sfd_col"], ref["sfd_col"])
    assert np.array_equal(got["d_col"], ref["d_col_code"])


def test_bf16_rounding_through_epilogue_bit_exact():
    """BF16 D = prob[m] * 2^-e(n) exactly (one nonzero product per dot), with
    prob on BF16 rounding ties (both parities) and one fp32 ulp either side
    of them: every BF16 code and the amax must match the oracle bit for bit
    (round to nearest, ties to even)."""
    rows, n, k = 1024, 256, 128
    case = synth.make_case("quant_gating_l4", seed=6, name="bf16_rounding", L=1, K=k, N=n, d="bf16",
                           force_counts=[rows])
    a = case.arrays
    a["a"][:] = 0
    a["a"][:, 0] = 0x38                                       # A[m, 0] = 1, rest 0
    a["sfa"][:] = 127
    a["b"][:] = 0
    e = (np.arange(n) % 32) // 2                              # 0..15 per 32-column block
    a["b"][0, :, 0] = 0x38
    a["sfb"][0, :, 0] = (127 - e).astype(np.uint8)            # B[n, 0] = 2^-e(n)
    a["sfb"][0, :, 1:] = 127
    a["alpha"][:] = 1.0
    rng = np.random.default_rng(66)
    hi16 = rng.integers(0x3F00, 0x3F80, rows).astype(np.uint32)   # values in [0.5, 1)
    lo16 = np.array([0x8000, 0x7FFF, 0x8001, 0x0000], dtype=np.uint32)[np.arange(rows) % 4]
    lo16[rows // 2:] = rng.integers(0, 1 << 16, rows - rows // 2).astype(np.uint32)
    a["prob"][:] = ((hi16 << 16) | lo16).view(np.float32)
    got = run_gpu(case)
    ref = oracle.grouped_gemm(case.problem, a)
    assert np.array_equal(got["d"].view(np.uint16), ref["d_bits"])
    assert np.array_equal(got["amax"].view(np.uint32), np.float32(ref["amax"]).view(np.uint32))


def test_deterministic_repeat():
    case = synth.make_case("fc1_swiglu_l8", seed=6, name="determinism", L=3, K=256, N=256,
                           routing=("topk", 300, 2))
    r1, r2 = run_gpu(case, times=2)
    for k in r1:
        assert np.array_equal(r1[k], r2[k]), k


def test_dswiglu_dprob_accumulates():
    """dprob is caller-zeroed and accumulated: a second call adds the same sums."""
    case = synth.make_case("dswiglu_bf16_l64", seed=7, name="dprob_acc", L=2, K=128, N=64,
                           routing=("topk", 100, 1))
    _announce(case)
    dev = pl.to_device(case.arrays)
    outs = pl.empty_outputs(case.problem)
    t = {**pl.inputs_for(case.problem, dev), **outs}
    mg.run(case.problem, t)
    torch.cuda.synchronize()
    once = outs["dprob"].cpu().numpy().copy()
    mg.run(case.problem, t)
    torch.cuda.synchronize()
    twice = outs["dprob"].cpu().numpy()
    np.testing.assert_allclose(twice, 2 * once, rtol=1e-6, atol=1e-30)


def test_check_offsets_on_device():
    case = synth.make_case("quant_gating_l4", seed=8, name="offsets", L=3, K=128, N=64,
                           force_counts=[10, 0, 300])
    _announce(case)
    po = torch.from_numpy(case.arrays["padded_offsets"]).cuda()
    prob = mg.make_problem(case.problem)
    assert mg.moegg_check_offsets(prob, po.data_ptr(), None) == 0
    bad = po.clone()
    bad[1] = 64                                   # not a multiple of 128
    assert mg.moegg_check_offsets(prob, bad.data_ptr(), None) == 1
    bad = po.clone()
    bad[2] = bad[1]                               # last != valid_m
    assert mg.moegg_check_offsets(prob, bad.data_ptr(), None) == 1


# ---------------------------------------------------------------------------
# full-size workloads: sampled 32-row blocks + properties at any size
# ---------------------------------------------------------------------------

FULL = ["fc1_swiglu_l8", "fc2_gating_l64_zipf", "srelu_tanh_fp4_l32", "dswiglu_bf16_l64", "fc1_swiglu_l64",
        "dswiglu_mxfp8_l64", "dsrelu_mxfp8_l32", "fc1_geglu_e5m2_l8", "dgeglu_mxfp8_l64"]


@pytest.mark.slow
def test_full_size_discrete_fc1_l64():
    """The L=64 FC1 workload with per-expert weight allocations: sampled rows
    against the oracle, every output bit-identical to the dense-weight run."""
    case = synth.make_case("fc1_swiglu_l64")
    got = run_gpu_discrete(case, fill=0x5A)
    rows = pick_row_blocks(case, nblocks=4)
    stats = check_case(case, got, rows)
    assert_same_as_dense(got, run_gpu(case, fill=0x5A))
    print(f"[gpu-case] fc1_swiglu_l64 discrete stats {stats}", flush=True)


def full_size_rows(case, nblocks=16):
    """Rows a full-size run is compared on, element by element: whole 32-row
    blocks spread over the groups (pick_row_blocks) plus every row of the
    largest group and of the last non-empty one (whole 32-row blocks too:
    groups are padded to multiples of 128)."""
    rows = set(pick_row_blocks(case, nblocks=nblocks).tolist())
    po = np.asarray(case.arrays["padded_offsets"], np.int64)
    starts = np.concatenate([[0], po[:-1]])
    sizes = po - starts
    for g in {int(np.argmax(sizes)), int(np.nonzero(sizes)[0][-1])}:
        rows.update(range(int(starts[g]), int(po[g])))
    return np.array(sorted(rows), np.int64)


@pytest.mark.slow
def test_full_size_every_row_fc1_l64():
    """The L=64 FC1 + SwiGLU workload that the benchmark reports, in its
    launch configuration (K-block plane scales), against the oracle on every
    row: D / D_col codes and both scale planes of each expert's rows, one
    group at a time."""
    case = synth.make_case("fc1_swiglu_l64")
    p = dict(case.problem, sf_layout="kplanes")
    dev = pl.to_device(case.arrays, sf_layout="kplanes", k=p["k"])
    outs = pl.empty_outputs(p, fill=0x5A)
    _announce(case)
    mg.run(p, {**pl.inputs_for(p, dev), **outs})
    torch.cuda.synchronize()
    got = pl.to_host(outs)
    po = np.asarray(case.arrays["padded_offsets"], np.int64)
    starts = np.concatenate([[0], po[:-1]])
    total = dict(elements=0, beyond_1ulp=0, scale_blocks=0, scale_boundary_mismatch=0, scale_acc_allowance=0)
    for g in range(p["num_groups"]):
        if po[g] == starts[g]:
            continue
        st = check_case(case, got, np.arange(starts[g], po[g]))
        for axis in ("d_row", "d_col"):
            for k in total:
                total[k] += st[axis][k]
    assert total["elements"] == 2 * int(case.problem["valid_m"]) * (p["n"] // 2)
    print(f"[gpu-case] fc1_swiglu_l64 every row {total}", flush=True)


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    case = synth.make_case(name)
    got = run_gpu(case, fill=0x5A)
    rows = full_size_rows(case)
    stats = check_case(case, got, rows)
    stats["rows_compared"] = len(rows)
    p = case.problem
    pad = ~case.row_valid
    if p["act"] in ("dswiglu", "dsrelu", "dgeglu"):
        # padding rows have A = 0, so R = 0: dC and dprob are (signed) zeros
        dpad = F.decode_e4m3(got["d"][pad]) if p["d_dtype"] == "e4m3" else decode_bf16(got["d"][pad])
        assert np.all(dpad == 0) and np.all(got["dprob"][pad] == 0)
    elif p["d_dtype"] == "bf16":
        d = decode_bf16(got["d"])
        assert np.all(d[pad] == 0)
        # every group against the oracle, one group's rows at a time: rule 1
        # on all of D and on each group's amax (0 for an empty group)
        po = np.asarray(case.arrays["padded_offsets"], np.int64)
        starts = np.concatenate([[0], po[:-1]])
        worst_d, ref_amax = 0.0, np.zeros(p["num_groups"])
        for g in range(p["num_groups"]):
            if po[g] == starts[g]:
                continue
            grows = np.arange(starts[g], po[g])
            ref_g = oracle.grouped_gemm(p, case.arrays, grows)
            worst_d = max(worst_d, rule1(d[grows], ref_g["d"], np.full(ref_g["d"].shape, g), f"D group {g}",
                                         make_envelope(case, ref_g)))
            ref_amax[g] = ref_g["amax"][g]
        stats["d_all_rows"] = worst_d
        stats["amax_all_groups"] = amax_rule(got["amax"], ref_amax)
    else:
        assert np.all(F.decode_e4m3(got["d"][pad]) == 0) and np.all(got["sfd_row"][pad] == 0)
    if p["d_dtype"] == "e4m3":
        # every element of the FP8 outputs: D and D_col consistent
        stats["row_col_consistent"] = row_col_consistency(got)
    bwd = p["act"] in ("dswiglu", "dsrelu", "dgeglu")
    if p.get("c_dtype") == "bf16" or (bwd and p["d_dtype"] == "bf16"):
        # every row of the BF16 C, or of the BF16 dC and dprob, against the
        # oracle, one group at a time
        po = np.asarray(case.arrays["padded_offsets"], np.int64)
        starts = np.concatenate([[0], po[:-1]])
        worst = {}
        for g in range(p["num_groups"]):
            if po[g] == starts[g]:
                continue
            grows = np.arange(starts[g], po[g])
            ref_g = oracle.grouped_gemm(p, case.arrays, grows)
            if p.get("c_dtype") == "bf16":
                r1 = rule1(decode_bf16(got["c"][grows]), ref_g["c"], np.full(ref_g["c"].shape, g), f"C group {g}")
                worst["c_all_rows"] = max(worst.get("c_all_rows", 0.0), r1)
            if bwd and p["d_dtype"] == "bf16":
                r1 = rule1(decode_bf16(got["d"][grows]), ref_g["dc"], np.full(ref_g["dc"].shape, g), f"dC group {g}",
                           make_envelope(case, ref_g))
                worst["dc_all_rows"] = max(worst.get("dc_all_rows", 0.0), r1)
                r1 = rule1(got["dprob"][grows], ref_g["dprob"], np.full(len(grows), g), f"dprob group {g}")
                worst["dprob_all_rows"] = max(worst.get("dprob_all_rows", 0.0), r1)
        stats.update(worst)
    print(f"[gpu-case] {name} stats {stats}", flush=True)
