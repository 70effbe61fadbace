"""The C++ oracle (oracle/cpp) against the numpy oracle, and planted mistakes
in the C++ oracle against the pins.  CPU only.

The two oracles are independent writings of the same definitions: neither
calls the other, and they agree here on every seeded recipe the GPU parity
tests use (float64 values to 1e-12 of the largest, every integer output,
scale byte, code and BF16 value exactly).  The pins in test_oracle_pins.py
and test_oracle_formats.py run on both; the mutants below show that those
pins catch a plausible mistake in each part of the C++ oracle."""
import importlib.util
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth
from cases import EDGE, SMALL
from oracle import cxx
from oracle import formats as F

_RECIPES = [(name, SMALL[name], 1000 + sorted(SMALL).index(name)) for name in SMALL] + \
           [(name, EDGE[name], 2000 + sorted(EDGE).index(name)) for name in EDGE]


def _compare(a, b):
    """Differences between two oracle result dicts (same keys required)."""
    msgs = []
    for k in sorted(set(a) | set(b)):
        if k == "acc":                       # numpy's unscaled sums; the C++ oracle reports C / R
            continue
        if k not in a or k not in b:
            msgs.append(f"{k} only in {'numpy' if k in a else 'C++'}")
            continue
        x, y = np.asarray(a[k]), np.asarray(b[k])
        if x.shape != y.shape:
            msgs.append(f"{k}: shape {x.shape} vs {y.shape}")
        elif x.dtype.kind == "f":
            scale = np.abs(x).max() if x.size else 0.0
            if x.size and np.abs(x - y).max() > 1e-12 * max(scale, 1e-300):
                msgs.append(f"{k}: float64 values differ by {np.abs(x - y).max():.3e} (max |ref| {scale:.3e})")
        elif k.endswith("_bits"):
            # BF16 values (the sign of a zero from a 0/1 mask may differ)
            if np.any(F.decode_bf16(x) != F.decode_bf16(y)):
                msgs.append(f"{k}: {int((F.decode_bf16(x) != F.decode_bf16(y)).sum())} BF16 values differ")
        elif np.any(x != y):
            msgs.append(f"{k}: {int((x != y).sum())} entries differ")
    return msgs


@pytest.mark.parametrize("name,recipe,seed", _RECIPES, ids=[r[0] for r in _RECIPES])
def test_cpp_oracle_matches_numpy_oracle(name, recipe, seed):
    base, over = recipe
    case = synth.make_case(base, seed=seed, name=name, **over)
    msgs = _compare(oracle.grouped_gemm(case.problem, case.arrays), cxx.grouped_gemm(case.problem, case.arrays))
    assert not msgs, f"{name}: " + "; ".join(msgs)


@pytest.mark.parametrize("base", ["fc1_swiglu_l8", "dswiglu_mxfp8_l64", "srelu_tanh_fp4_l32"])
def test_cpp_oracle_matches_on_sampled_rows_of_full_workloads(base):
    """Full-size workloads on a few whole 32-row blocks (the way the full-size
    GPU checks sample them), including the column quantisation."""
    case = synth.make_case(base)
    vm = case.problem["valid_m"]
    blocks = np.linspace(0, vm // 32 - 1, 3).astype(np.int64)
    rows = (blocks[:, None] * 32 + np.arange(32)).reshape(-1)
    msgs = _compare(oracle.grouped_gemm(case.problem, case.arrays, rows),
                    cxx.grouped_gemm(case.problem, case.arrays, rows))
    assert not msgs, f"{base}: " + "; ".join(msgs)


# ---------------------------------------------------------------------------
# planted mistakes: each mutant of oracle.cpp must fail at least one pin
# ---------------------------------------------------------------------------

import test_oracle_formats as PF  # noqa: E402
import test_oracle_pins as PP  # noqa: E402

_W = {c["name"]: c for c in PP._CASES}

# (name, text in oracle.cpp, replacement, pins that must catch it)
_MUTANTS = [
    ("swiglu_block_order",
     "const double xv = c[64 * b + i], g = c[64 * b + 32 + i];",
     "const double g = c[64 * b + i], xv = c[64 * b + 32 + i];",
     [lambda O: PP.test_worked_example(_W["W2_swiglu_order"], O), PP.test_swiglu_closed_forms]),
    ("e8m0_rounds_down",
     "const int e = frac == 0.5f ? ex - 1 : ex;",
     "const int e = ex - 1;",
     [lambda O: PP.test_worked_example(_W["W1_gating_quant"], O),
      lambda O: PP.test_quantization_invariants(1.0, O)]),
    ("backward_alpha_not_squared",
     "const double scale = bwd ? alpha * alpha : alpha;",
     "const double scale = alpha;",
     [PP.test_dswiglu_alpha_squared_and_beta_placement, PP.test_dsrelu_through_the_gemm_closed_form]),
    ("dswiglu_gate_derivative_sign",
     "d[64 * b + 32 + i] = c[j] * pr * xv * s * (1.0 + g * (1.0 - s));",
     "d[64 * b + 32 + i] = c[j] * pr * xv * s * (1.0 - g * (1.0 - s));",
     [PP.test_dswiglu_matches_finite_differences]),
    ("bf16_truncates",
     "const double r = std::ldexp(std::nearbyint(std::ldexp(v, -qe)), qe);",
     "const double r = std::ldexp(std::trunc(std::ldexp(v, -qe)), qe);",
     [PF.test_bf16_encode_vs_torch]),
    ("e4m3_subnormal_exponent",
     "const double mag = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);",
     "const double mag = e == 0 ? std::ldexp(m / 8.0, -7) : std::ldexp(1.0 + m / 8.0, e - 7);",
     [PF.test_e4m3_decode_all_codes_vs_torch]),
    ("row_group_boundary",
     "while (g < L && rows[i] >= in->padded_offsets[g]) ++g;",
     "while (g < L && rows[i] > in->padded_offsets[g]) ++g;",
     [lambda O: PP.test_row_group_map_bit_exact([0, 3, 0, 2, 0], O)]),
    ("srelu_clamp_dropped",
     "if (p.srelu_s > 0) r = p.srelu_s * std::min(std::tanh(r / p.srelu_s), 1.0);",
     "if (p.srelu_s > 0) r = std::min(std::tanh(r / p.srelu_s), 1.0);",
     [PP.test_srelu_properties]),
    ("dsrelu_derivative_cancels",
     "fp = 2.0 * cv / (ch * ch);",
     "fp = 2.0 * cv * (1.0 - t * t);",
     [PP.test_dsrelu_derivative_in_the_saturated_clamp]),
    ("dgeglu_up_mask_dropped",
     "d[64 * b + 32 + i] = (p.clamp_min <= up && up <= p.clamp_max) ? c[j] * pr * gc * s : 0.0;",
     "d[64 * b + 32 + i] = c[j] * pr * gc * s;",
     [PP.test_dgeglu_clamp_masks_closed_form]),
]


def _mutant_module(tmp_path, name, old, new):
    src = open(cxx.SOURCES[0]).read()
    assert src.count(old) == 1, f"mutation site of {name} not found once"
    d = tmp_path / name
    d.mkdir()
    shutil.copy(os.path.join(cxx.HERE, "oracle.h"), d / "oracle.h")
    (d / "oracle.cpp").write_text(src.replace(old, new))
    lib = d / "liboracle.so"
    r = subprocess.run(["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                        "-o", str(lib), str(d / "oracle.cpp")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    spec = importlib.util.spec_from_file_location(f"cxx_{name}", cxx.__file__)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.LIB_PATH, mod._lib = str(lib), None
    return mod


@pytest.mark.parametrize("name,old,new,pins", _MUTANTS, ids=[m[0] for m in _MUTANTS])
def test_planted_mistake_in_cpp_oracle_is_caught(tmp_path, name, old, new, pins):
    mod = _mutant_module(tmp_path, name, old, new)
    caught = 0
    for pin in pins:
        try:
            pin(mod)
        except AssertionError:
            caught += 1
    assert caught, f"no pin caught the planted mistake {name}"


# ---------------------------------------------------------------------------
# the C++ oracle under the address and undefined-behaviour sanitizers
# ---------------------------------------------------------------------------

_SAN_RECIPES = ["swiglu_fp8_e4m3", "srelu_fp4_tanh_e4m3", "dswiglu_bf16", "dgeglu_e5m2_bf16_amax",
                "dsrelu_mxfp4_e4m3_n288", "geglu_fp4_e4m3_c"]


@pytest.fixture(scope="module")
def sanitized_driver(tmp_path_factory):
    """oracle.cpp + run_case.cpp built with -fsanitize=address,undefined (no
    OpenMP), so that an out-of-bounds access or undefined operation in the
    oracle aborts the run."""
    d = tmp_path_factory.mktemp("asan")
    exe = d / "run_case"
    r = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                        "-o", str(exe), os.path.join(cxx.HERE, "oracle.cpp"), os.path.join(cxx.HERE, "run_case.cpp")],
                       capture_output=True, text=True)
    if r.returncode:
        pytest.skip("no sanitizer runtime for g++ here: " + r.stderr[-300:])
    return exe


@pytest.mark.parametrize("name", _SAN_RECIPES)
def test_cpp_oracle_under_sanitizers(sanitized_driver, tmp_path, name):
    base, over = SMALL[name]
    case = synth.make_case(base, seed=1000 + sorted(SMALL).index(name), name=name, **over)
    p, arr = case.problem, case.arrays
    rows = np.arange(p["valid_m"], dtype=np.int64)
    kv = cxx._problem(p)
    nc = float(np.asarray(arr["norm_const"], np.float32).reshape(-1)[0]) if "norm_const" in arr else 1.0
    with open(tmp_path / "problem.txt", "w") as f:
        for key in ("num_groups", "valid_m", "n", "k", "ab", "act", "d_fp8", "c_out", "srelu_s", "glu_gamma",
                    "geglu_alpha", "linear_offset", "clamp_min", "clamp_max"):
            f.write(f"{key} {float(getattr(kv, key))!r}\n")
        f.write(f"norm_const {nc!r}\nnrows {len(rows)}\n")
    code_t = np.uint16 if p["ab_dtype"] == "bf16" else np.uint8
    files = {"a": ("a", code_t), "sfa": ("sfa", np.uint8), "b": ("b", code_t), "sfb": ("sfb", np.uint8),
             "po": ("padded_offsets", np.int32), "alpha": ("alpha", np.float32), "beta": ("beta", np.float32),
             "prob": ("prob", np.float32), "c_in": ("c_in", np.uint16)}
    for fname, (key, dt) in files.items():
        if arr.get(key) is not None:
            np.ascontiguousarray(arr[key], dtype=dt).tofile(tmp_path / f"{fname}.bin")
    rows.tofile(tmp_path / "rows.bin")
    r = subprocess.run([str(sanitized_driver), str(tmp_path)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"sanitized oracle failed on {name}:\n{r.stderr[-3000:]}"
    ref = cxx.grouped_gemm(p, arr)
    m, n, no = len(rows), p["n"], cxx.n_out(p)
    bwd = p["act"] in ("dswiglu", "dsrelu", "dgeglu")
    got_d = np.fromfile(tmp_path / "d.out", np.float64).reshape(m, no)
    assert np.array_equal(got_d, ref["dc" if bwd else "d"])
    assert np.array_equal(np.fromfile(tmp_path / "cr.out", np.float64).reshape(m, n), ref["r" if bwd else "c"])
    if "d_code" in ref:
        assert np.array_equal(np.fromfile(tmp_path / "d_code.out", np.uint8).reshape(m, no), ref["d_code"])
        assert np.array_equal(np.fromfile(tmp_path / "sfd_row.out", np.uint8).reshape(m, no // 32), ref["sfd_row"])
    if "amax2" in ref or "amax" in ref:
        want = ref.get("amax2", ref.get("amax"))
        assert np.array_equal(np.fromfile(tmp_path / "amax.out", np.float64).reshape(want.shape), want)
