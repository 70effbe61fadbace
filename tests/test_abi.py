"""C-ABI checks that need no GPU: the library loads, exports every function
include/moegg.h declares, and its host-side validation returns the right
status for every rule, before any HIP call (no device memory is touched:
the pointers below are fake, aligned integers)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moegg.h")

import moe_grouped_block_amd as mg  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _built():
    if not os.path.exists(mg.lib_path):
        from moe_grouped_block_amd import build
        build.build()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*[A-Za-z_][A-Za-z0-9_ \*]*?\b(moegg_[a-z_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_function():
    names = _declared_functions()
    assert {"moegg_check", "moegg_run", "moegg_check_offsets", "moegg_n_out", "moegg_status_string",
            "moegg_last_error", "moegg_abi_version", "moegg_set_grid_limit",
            "moegg_sf_to_kplanes"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", mg.lib_path], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moegg_[a-z_]+)\b", out))
    assert set(names) <= exported, set(names) - exported
    lib = ctypes.CDLL(mg.lib_path)
    for n in names:
        getattr(lib, n)


def test_version_and_strings():
    assert mg.moegg_abi_version() == 5 == mg.ABI_VERSION
    for code, name in mg.STATUS.items():
        assert mg.moegg_status_string(code) == name
    assert mg.moegg_status_string(99) == "MOEGG_UNKNOWN_STATUS"


def test_struct_layout_matches_header():
    # problem: 2 x int32, int64, 6 x int32, float -> 44 bytes, padded to 48
    assert ctypes.sizeof(mg.moegg_problem) == 72
    assert mg.moegg_problem.valid_m.offset == 8
    assert mg.moegg_problem.sf_layout.offset == 64
    assert ctypes.sizeof(mg.moegg_args) == 19 * 8
    assert mg.moegg_args.b_ptrs.offset == 17 * 8 and mg.moegg_args.sfb_ptrs.offset == 18 * 8


FAKE = 0x7F0000000000            # 16-byte aligned, never dereferenced by moegg_check


def _ptrs(names):
    return {n: FAKE + 0x1000 * i for i, n in enumerate(names)}


def _base(kind):
    if kind == "swiglu_e4m3":
        p = dict(num_groups=8, m_aligned=128, valid_m=8704, n=2816, k=2048, ab_dtype="e4m3",
                 c_dtype=None, d_dtype="e4m3", act="swiglu", srelu_tanh_s=0.0)
        t = _ptrs(["a", "b", "sfa", "sfb", "padded_offsets", "alpha", "prob", "norm_const",
                   "d", "d_col", "sfd_row", "sfd_col"])
    elif kind == "gating_bf16":
        p = dict(num_groups=4, m_aligned=128, valid_m=1024, n=512, k=512, ab_dtype="e4m3",
                 c_dtype=None, d_dtype="bf16", act="none")
        t = _ptrs(["a", "b", "sfa", "sfb", "padded_offsets", "alpha", "prob", "d", "amax"])
    elif kind == "srelu_fp4":
        p = dict(num_groups=32, m_aligned=128, valid_m=34560, n=4096, k=4096, ab_dtype="e2m1x2",
                 c_dtype="bf16", d_dtype="e4m3", act="srelu", srelu_tanh_s=8.0)
        t = _ptrs(["a", "b", "sfa", "sfb", "padded_offsets", "alpha", "prob", "norm_const", "c",
                   "d", "d_col", "sfd_row", "sfd_col"])
    else:
        p = dict(num_groups=64, m_aligned=128, valid_m=102144, n=1408, k=2048, ab_dtype="bf16",
                 c_dtype=None, d_dtype="bf16", act="dswiglu")
        t = _ptrs(["a", "b", "padded_offsets", "alpha", "prob", "beta", "c_in", "d", "dprob"])
    return p, t


def _status(p, t):
    return mg.moegg_check(mg.make_problem(p), mg.make_args(t))


@pytest.mark.parametrize("kind", ["swiglu_e4m3", "gating_bf16", "srelu_fp4", "dswiglu"])
def test_valid_configs_pass(kind):
    p, t = _base(kind)
    assert _status(p, t) == 0, mg.moegg_last_error()


OK, INVALID, MISALIGNED, NOT_SUPPORTED = 0, 1, 2, 3

CASES = [
    # (base, problem overrides, tensor overrides, expected status)
    ("gating_bf16", dict(num_groups=0), {}, INVALID),
    ("gating_bf16", dict(sf_layout=1), {}, OK),                        # K-block planes
    ("gating_bf16", dict(sf_layout=2), {}, INVALID),                   # unknown scale layout
    ("gating_bf16", dict(num_groups=1025), {}, INVALID),
    ("gating_bf16", dict(n=0), {}, INVALID),
    ("gating_bf16", dict(valid_m=-128), {}, INVALID),
    ("gating_bf16", dict(valid_m=1000), {}, INVALID),                  # not a multiple of m_aligned
    ("gating_bf16", dict(m_aligned=48), {}, INVALID),
    ("gating_bf16", dict(m_aligned=64, valid_m=1024), {}, NOT_SUPPORTED),
    ("gating_bf16", dict(k=500), {}, INVALID),                         # K % 32
    ("gating_bf16", dict(k=544), {}, NOT_SUPPORTED),                   # FP8 step of 128
    ("srelu_fp4", dict(k=4096 + 128), {}, NOT_SUPPORTED),              # FP4 step of 256
    ("gating_bf16", dict(n=500), {}, NOT_SUPPORTED),                   # N % 32
    ("swiglu_e4m3", dict(n=2816 + 32), {}, INVALID),                   # SwiGLU N % 64
    ("dswiglu", dict(n=1408 + 16), {}, INVALID),                       # dGLU N % 32
    ("dswiglu", dict(ab_dtype="e4m3"), dict(sfa=FAKE, sfb=FAKE), INVALID),            # MX + bf16 dC needs amax
    ("dswiglu", dict(ab_dtype="e4m3"), dict(sfa=FAKE, sfb=FAKE, amax=FAKE), OK),
    ("dswiglu", dict(ab_dtype="e4m3", d_dtype="e4m3"),
     dict(sfa=FAKE, sfb=FAKE, d_col=FAKE + 0x40000, sfd_row=FAKE + 0x50000, sfd_col=FAKE + 0x60000,
          norm_const=FAKE + 0x70000), OK),
    ("dswiglu", dict(ab_dtype="e4m3", d_dtype="e4m3"),
     dict(sfa=FAKE, sfb=FAKE, d_col=FAKE + 0x40000, sfd_row=FAKE + 0x50000, sfd_col=FAKE + 0x60000), INVALID),
    ("dswiglu", {}, dict(amax=FAKE), INVALID),                                   # BF16 operands: no amax
    # sReLU backward: c_in (N wide) and dprob, no beta
    ("dswiglu", dict(act="dsrelu"), dict(beta=None), OK),
    ("dswiglu", dict(act="dsrelu"), {}, INVALID),                                # beta given
    ("dswiglu", dict(act="dsrelu"), dict(beta=None, c_in=None), INVALID),
    ("dswiglu", dict(act="dsrelu", ab_dtype="e4m3"), dict(beta=None, sfa=FAKE, sfb=FAKE, amax=FAKE), OK),
    ("dswiglu", dict(act="dsrelu", d_dtype="e4m3"), dict(beta=None), NOT_SUPPORTED),   # BF16 ops: bf16 dC
    ("gating_bf16", {}, dict(prob=None), INVALID),                     # prob required
    ("gating_bf16", {}, dict(amax=None), INVALID),                     # amax for bf16 D
    ("gating_bf16", {}, dict(sfa=None), INVALID),
    ("gating_bf16", {}, dict(alpha=None), INVALID),
    ("swiglu_e4m3", {}, dict(sfd_col=None), INVALID),                  # SFD trio all-or-none
    ("swiglu_e4m3", {}, dict(norm_const=None), INVALID),
    ("swiglu_e4m3", {}, dict(d_col=None), INVALID),
    ("swiglu_e4m3", {}, dict(amax=FAKE), INVALID),
    ("gating_bf16", {}, dict(norm_const=FAKE), INVALID),
    ("gating_bf16", {}, dict(a=FAKE + 8), MISALIGNED),
    ("gating_bf16", {}, dict(d=FAKE + 4), MISALIGNED),
    ("gating_bf16", {}, dict(prob=FAKE + 2), MISALIGNED),
    ("srelu_fp4", dict(c_dtype=None), {}, INVALID),                    # c given without c_dtype
    ("srelu_fp4", {}, dict(c=None), INVALID),
    ("srelu_fp4", dict(srelu_tanh_s=-1.0), {}, INVALID),
    ("srelu_fp4", dict(srelu_tanh_s=float("inf")), {}, INVALID),
    ("dswiglu", {}, dict(beta=None), INVALID),
    ("dswiglu", {}, dict(c_in=None), INVALID),
    ("dswiglu", {}, dict(dprob=None), INVALID),
    ("dswiglu", dict(d_dtype="e4m3"), {}, NOT_SUPPORTED),
    ("gating_bf16", {}, dict(beta=FAKE), INVALID),                     # dSwiGLU-only input
    ("gating_bf16", dict(ab_dtype="bf16"), {}, INVALID),               # sfa/sfb with BF16 operands
    ("gating_bf16", dict(valid_m=2 ** 31), {}, NOT_SUPPORTED),
    ("gating_bf16", dict(n=(1 << 20) + 32), {}, NOT_SUPPORTED),            # epilogue offsets are 32-bit
    ("gating_bf16", dict(n=1 << 20), {}, OK),
    # discrete weights (b_ptrs / sfb_ptrs instead of b / sfb)
    ("gating_bf16", {}, dict(b=None, sfb=None, b_ptrs=FAKE + 0x20000, sfb_ptrs=FAKE + 0x21000), OK),
    ("dswiglu", {}, dict(b=None, b_ptrs=FAKE + 0x20000), OK),
    ("gating_bf16", {}, dict(b_ptrs=FAKE + 0x20000), INVALID),               # both b and b_ptrs
    ("gating_bf16", {}, dict(b=None), INVALID),                              # neither
    ("gating_bf16", {}, dict(b=None, b_ptrs=FAKE + 0x20000), INVALID),       # dense sfb with b_ptrs
    ("gating_bf16", {}, dict(b=None, sfb=None, b_ptrs=FAKE + 0x20000), INVALID),   # MX without sfb_ptrs
    ("gating_bf16", {}, dict(sfb_ptrs=FAKE + 0x21000), INVALID),             # sfb_ptrs with dense b
    ("dswiglu", {}, dict(b=None, b_ptrs=FAKE + 0x20000, sfb_ptrs=FAKE + 0x21000), INVALID),   # BF16 + sfb_ptrs
    ("gating_bf16", {}, dict(b=None, sfb=None, b_ptrs=FAKE + 0x20004, sfb_ptrs=FAKE + 0x21000), MISALIGNED),
    # E5M2 operands: the E4M3 layout and K step
    ("swiglu_e4m3", dict(ab_dtype="e5m2"), {}, OK),
    ("swiglu_e4m3", dict(ab_dtype="e5m2", k=2048 + 64), {}, NOT_SUPPORTED),
    ("swiglu_e4m3", dict(ab_dtype="e5m2"), dict(sfb=None), INVALID),
    # GeGLU forward: pairs of 32 columns, finite constants, ordered clamps
    ("swiglu_e4m3", dict(act="geglu", glu_clamp_min=-7.0, glu_clamp_max=7.0), {}, OK),
    ("swiglu_e4m3", dict(act="geglu", ab_dtype="e5m2"), {}, OK),
    ("swiglu_e4m3", dict(act="geglu", n=2816 + 32), {}, INVALID),
    ("swiglu_e4m3", dict(act="geglu", glu_clamp_min=1.0, glu_clamp_max=-1.0), {}, INVALID),
    ("swiglu_e4m3", dict(act="geglu", glu_clamp_min=float("nan")), {}, INVALID),
    ("swiglu_e4m3", dict(act="geglu", geglu_alpha=float("inf")), {}, INVALID),
    ("swiglu_e4m3", dict(act="geglu", linear_offset=float("nan")), {}, INVALID),
    ("swiglu_e4m3", dict(act="geglu", glu_gamma=float("-inf")), {}, INVALID),
    ("gating_bf16", dict(act="geglu"), {}, OK),                               # bf16 D + amax
    # dGeGLU backward: c_in 2N wide, dprob, no beta; amax (L, 2) for MX operands and a bf16 dC
    ("dswiglu", dict(act="dgeglu"), dict(beta=None), OK),
    ("dswiglu", dict(act="dgeglu"), {}, INVALID),                                # beta given
    ("dswiglu", dict(act="dgeglu"), dict(beta=None, c_in=None), INVALID),
    ("dswiglu", dict(act="dgeglu"), dict(beta=None, dprob=None), INVALID),
    ("dswiglu", dict(act="dgeglu", glu_clamp_min=7.0, glu_clamp_max=-7.0), dict(beta=None), INVALID),
    ("dswiglu", dict(act="dgeglu", ab_dtype="e4m3"), dict(beta=None, sfa=FAKE, sfb=FAKE, amax=FAKE), OK),
    ("dswiglu", dict(act="dgeglu", ab_dtype="e5m2"), dict(beta=None, sfa=FAKE, sfb=FAKE, amax=FAKE), OK),
    ("dswiglu", dict(act="dgeglu", ab_dtype="e4m3"), dict(beta=None, sfa=FAKE, sfb=FAKE), INVALID),
    ("dswiglu", dict(act="dgeglu", ab_dtype="e4m3", d_dtype="e4m3"),
     dict(beta=None, sfa=FAKE, sfb=FAKE, d_col=FAKE + 0x40000, sfd_row=FAKE + 0x50000,
          sfd_col=FAKE + 0x60000, norm_const=FAKE + 0x70000), OK),
    ("dswiglu", dict(act="dgeglu", d_dtype="e4m3"), dict(beta=None), NOT_SUPPORTED),   # BF16 ops: bf16 dC
    ("dswiglu", dict(act=7), {}, INVALID),
]


@pytest.mark.parametrize("base,pov,tov,expect", CASES)
def test_validation_rules(base, pov, tov, expect):
    p, t = _base(base)
    p.update(pov)
    t.update(tov)
    t = {k: v for k, v in t.items() if v is not None}
    st = _status(p, t)
    assert st == expect, (st, mg.moegg_last_error())
    if expect != OK:
        assert mg.moegg_last_error() != ""


def test_run_rejects_before_any_hip_call():
    # an invalid call must return its status without touching the (absent) GPU
    p, t = _base("gating_bf16")
    t.pop("prob")
    st = mg.moegg_run(mg.make_problem(p), mg.make_args(t), None)
    assert st == INVALID


def test_null_structs():
    lib = ctypes.CDLL(mg.lib_path)
    lib.moegg_check.restype = ctypes.c_int
    assert lib.moegg_check(None, None) == INVALID
    assert lib.moegg_n_out.restype != 0  # attribute exists


def test_n_out():
    for act, n, expect in [("none", 512, 512), ("swiglu", 2816, 1408), ("srelu", 4096, 4096),
                           ("dswiglu", 1408, 2816), ("dsrelu", 4096, 4096), ("geglu", 2816, 1408),
                           ("dgeglu", 1408, 2816)]:
        p, _ = _base("gating_bf16")
        p.update(act=act, n=n)
        assert mg.moegg_n_out(mg.make_problem(p)) == expect


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    # no fallback path: a missing library is an error, not a silent CPU run
    monkeypatch.setattr(mg, "lib_path", str(tmp_path / "absent.so"))
    monkeypatch.setattr(mg, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        mg.moegg_abi_version()


def test_binding_rejects_a_library_of_another_abi(tmp_path, monkeypatch):
    # a stale build (an older struct layout) must not be called with these structs
    monkeypatch.setattr(mg, "_lib", None)
    monkeypatch.setattr(mg, "ABI_VERSION", mg.ABI_VERSION + 1)
    with pytest.raises(RuntimeError, match="rebuild"):
        mg.moegg_abi_version()
    monkeypatch.setattr(mg, "_lib", None)


def test_grid_limit_hook_round_trips():
    """The testing hook returns the previous cap; 0 and negative values clear it."""
    prev = mg.moegg_set_grid_limit(3)
    try:
        assert mg.moegg_set_grid_limit(7) == 3
        assert mg.moegg_set_grid_limit(-5) == 7
        assert mg.moegg_set_grid_limit(0) == 0
    finally:
        mg.moegg_set_grid_limit(prev)


def test_sf_to_kplanes_rejects_bad_arguments_before_any_launch():
    """Argument rules of the scale-layout conversion (no device work: each
    case fails validation, and rows == 0 enqueues nothing)."""
    assert mg.moegg_sf_to_kplanes(FAKE, FAKE + 0x100000, 10, 200, None) == INVALID       # k % 128
    assert mg.moegg_sf_to_kplanes(FAKE, FAKE + 0x100000, -1, 256, None) == INVALID        # rows < 0
    assert mg.moegg_sf_to_kplanes(FAKE + 4, FAKE + 0x100000, 10, 256, None) == MISALIGNED
    assert mg.moegg_sf_to_kplanes(FAKE, FAKE + 8, 10, 256, None) == MISALIGNED
    assert mg.moegg_sf_to_kplanes(FAKE, FAKE + 16, 10, 256, None) == INVALID             # overlap
    assert mg.moegg_sf_to_kplanes(None, FAKE, 10, 256, None) == INVALID
    assert mg.moegg_sf_to_kplanes(FAKE, FAKE + 0x100000, 0, 256, None) == OK              # nothing to do
