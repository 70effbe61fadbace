"""Pins of the oracles' GEMM, row->group map, epilogues and quantisation
against closed forms, brute force, finite differences and the hand-worked
examples in tests/golden/worked_examples.yaml.  Every pin runs on both
oracles: the numpy one (``oracle.grouped``) and the C++ one (``oracle/cpp``,
through ``oracle.cxx``).  CPU only."""
import itertools
import math
import os

import numpy as np
import pytest
import yaml

import oracle
from oracle import formats as F
from oracle import grouped as G

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.yaml")
RCP_MAX_E4M3 = np.float32(1.0) / np.float32(448.0)


class _Numpy:
    """The numpy oracle under the names the pins use."""
    grouped_gemm = staticmethod(oracle.grouped_gemm)
    swiglu, srelu, geglu = staticmethod(G.swiglu), staticmethod(G.srelu), staticmethod(G.geglu)
    dswiglu, dsrelu, dgeglu = staticmethod(G.dswiglu), staticmethod(G.dsrelu), staticmethod(G.dgeglu)
    quantize_rows, quantize_cols = staticmethod(G.quantize_rows), staticmethod(G.quantize_cols)
    e8m0_block_scale = staticmethod(G.e8m0_block_scale)


@pytest.fixture(params=["numpy", "cpp"])
def O(request):
    """Each pin runs against both oracles."""
    if request.param == "numpy":
        return _Numpy
    from oracle import cxx
    return cxx


# ---------------------------------------------------------------------------
# helpers that build inputs from explicit codes
# ---------------------------------------------------------------------------

def _problem(L, valid_m, n, k, ab="e4m3", act="none", d="bf16", c=None, s=0.0):
    return dict(num_groups=L, valid_m=valid_m, n=n, k=k, ab_dtype=ab, c_dtype=c, d_dtype=d,
                act=act, srelu_tanh_s=s)


def _const_mx(rows, k, code, byte, fp4=False):
    kb = k // 2 if fp4 else k
    return (np.full((rows, kb), code, np.uint8), np.full((rows, k // 32), byte, np.uint8))


# ---------------------------------------------------------------------------
# P-b: dequantisation + GEMM
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fp4", [False, True])
@pytest.mark.parametrize("sa,sb,alpha", [(127, 127, 1.0), (130, 120, 0.5), (100, 140, 4.0)])
def test_all_ones_power_of_two_scales_exact(fp4, sa, sb, alpha, O):
    k, n, m = 256, 64, 8
    one = 0x22 if fp4 else 0x38
    a, sfa = _const_mx(m, k, one, sa, fp4)
    b, sfb = _const_mx(n, k, one, sb, fp4)
    ab = "e2m1x2" if fp4 else "e4m3"
    arr = dict(a=a, sfa=sfa, b=b[None], sfb=sfb[None], padded_offsets=np.array([m], np.int32),
               alpha=np.array([alpha], np.float32), prob=np.ones(m, np.float32))
    out = O.grouped_gemm(_problem(1, m, n, k, ab=ab), arr)
    expect = k * alpha * 2.0 ** (sa - 127 + sb - 127)
    assert np.all(out["c"] == expect)
    assert np.all(out["d"] == expect)


def _brute_force(problem, arr):
    """Triple loop in pure Python over decoded scalars (no numpy matmul)."""
    m, n, k = problem["valid_m"], problem["n"], problem["k"]
    fp4 = problem["ab_dtype"] == "e2m1x2"

    def elem(codes, sf, r, kk):
        if fp4:
            byte = int(codes[r, kk // 2])
            nib = byte & 0xF if kk % 2 == 0 else byte >> 4
            v = float(F.decode_e2m1(nib))
        else:
            v = float(F.decode_e4m3(int(codes[r, kk])))
        return v * 2.0 ** (int(sf[r, kk // 32]) - 127)

    po = list(arr["padded_offsets"])
    out = np.zeros((m, n))
    for r in range(m):
        g = next(i for i, e in enumerate(po) if r < e)
        for j in range(n):
            s = 0.0
            for kk in range(k):
                s += elem(arr["a"], arr["sfa"], r, kk) * elem(arr["b"][g], arr["sfb"][g], j, kk)
            out[r, j] = float(arr["alpha"][g]) * s
    return out


@pytest.mark.parametrize("ab", ["e4m3", "e2m1x2"])
def test_gemm_vs_brute_force_tiny(ab, O):
    rng = np.random.default_rng(3)
    m, n, k, L = 6, 5 * 1, 64, 2
    fp4 = ab == "e2m1x2"
    kb = k // 2 if fp4 else k
    if fp4:
        a = rng.integers(0, 256, (m, kb), dtype=np.uint8)
        b = rng.integers(0, 256, (L, n, kb), dtype=np.uint8)
    else:
        # random finite E4M3 codes (avoid the NaN code 0x7f / 0xff)
        a = rng.integers(0, 0x7F, (m, kb), dtype=np.uint8) | (rng.integers(0, 2, (m, kb), dtype=np.uint8) << 7)
        b = rng.integers(0, 0x7F, (L, n, kb), dtype=np.uint8) | (rng.integers(0, 2, (L, n, kb), dtype=np.uint8) << 7)
    arr = dict(a=a, b=b, sfa=rng.integers(120, 135, (m, k // 32), dtype=np.uint8),
               sfb=rng.integers(120, 135, (L, n, k // 32), dtype=np.uint8),
               padded_offsets=np.array([4, 6], np.int32),
               alpha=np.array([0.75, -1.5], np.float32), prob=np.ones(m, np.float32))
    prob = _problem(L, m, n, k, ab=ab)
    out = O.grouped_gemm(prob, arr)
    ref = _brute_force(prob, arr)
    np.testing.assert_allclose(out["c"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_one_hot_b_selects_a_column(O):
    rng = np.random.default_rng(5)
    m, k = 4, 64
    n = 32
    a = rng.integers(0, 0x7F, (m, k), dtype=np.uint8)
    sfa = rng.integers(120, 135, (m, k // 32), dtype=np.uint8)
    b = np.zeros((1, n, k), np.uint8)
    for j in range(n):
        b[0, j, 2 * j + 1] = 0x38                       # column j picks K index 2j+1
    arr = dict(a=a, sfa=sfa, b=b, sfb=np.full((1, n, k // 32), 127, np.uint8),
               padded_offsets=np.array([m], np.int32), alpha=np.array([2.0], np.float32),
               prob=np.ones(m, np.float32))
    out = O.grouped_gemm(_problem(1, m, n, k), arr)
    vals = F.decode_e4m3(a) * np.repeat(2.0 ** (sfa.astype(np.float64) - 127), 32, axis=1)
    assert np.array_equal(out["c"], 2.0 * vals[:, 1::2][:, :n])


# ---------------------------------------------------------------------------
# P-c: row -> group map (alpha_g = 2^g makes each row's group visible)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("counts", [
    [0, 3, 0, 2, 0],         # empty first, middle and last groups
    [1, 1, 1],               # single-row groups
    [5],
    [0, 0, 4],
])
def test_row_group_map_bit_exact(counts, O):
    pad = 4
    L = len(counts)
    padded = [((c + pad - 1) // pad) * pad for c in counts]
    po = np.cumsum(padded).astype(np.int32)
    m = int(po[-1])
    k, n = 32, 32
    a = np.zeros((m, k), np.uint8)
    start = 0
    for c, p in zip(counts, padded):
        a[start:start + c] = 0x38                      # routed rows carry 1.0; padding 0
        start += p
    arr = dict(a=a, sfa=np.full((m, 1), 127, np.uint8), b=np.full((L, n, k), 0x38, np.uint8),
               sfb=np.full((L, n, 1), 127, np.uint8), padded_offsets=po,
               alpha=(2.0 ** np.arange(L)).astype(np.float32), prob=np.ones(m, np.float32))
    out = O.grouped_gemm(_problem(L, m, n, k), arr)
    start = 0
    for g, (c, p) in enumerate(zip(counts, padded)):
        blk = out["c"][start:start + p]
        assert np.all(blk[:c] == 32 * 2.0 ** g)
        assert np.all(blk[c:] == 0)
        assert np.all(out["group"][start:start + p] == g)
        start += p
    # amax of an empty group is 0, of a non-empty group the brute-force max
    for g, c in enumerate(counts):
        assert out["amax"][g] == (32 * 2.0 ** g if c else 0.0)


# ---------------------------------------------------------------------------
# P-d / P-h: gating and amax
# ---------------------------------------------------------------------------

def test_gating_exact_and_amax_brute_force(O):
    rng = np.random.default_rng(9)
    m, n, k = 8, 64, 64
    arr = dict(a=np.full((m, k), 0x38, np.uint8), sfa=np.full((m, 2), 127, np.uint8),
               b=np.full((2, n, k), 0x38, np.uint8), sfb=np.full((2, n, 2), 126, np.uint8),
               padded_offsets=np.array([3, 8], np.int32), alpha=np.array([1.0, 0.25], np.float32),
               prob=rng.random(m).astype(np.float32))
    out = O.grouped_gemm(_problem(2, m, n, k), arr)
    grp = np.array([0, 0, 0, 1, 1, 1, 1, 1])
    expect = k * 0.5 * np.array([1.0, 0.25])[grp] * arr["prob"].astype(np.float64)
    assert np.array_equal(out["d"], np.repeat(expect[:, None], n, axis=1))
    for g in range(2):
        bf = max(abs(out["d"][r, j]) for r in range(m) for j in range(n) if grp[r] == g)
        assert out["amax"][g] == bf


def test_random_amax_is_brute_force_max(O):
    rng = np.random.default_rng(12)
    m, n, k, L = 12, 64, 64, 3
    arr = dict(a=rng.integers(0, 0x7F, (m, k), dtype=np.uint8) | 0x80 * rng.integers(0, 2, (m, k), dtype=np.uint8),
               sfa=rng.integers(125, 130, (m, 2), dtype=np.uint8),
               b=rng.integers(0, 0x7F, (L, n, k), dtype=np.uint8), sfb=rng.integers(125, 130, (L, n, 2), dtype=np.uint8),
               padded_offsets=np.array([4, 4, 12], np.int32), alpha=np.array([1, 2, 3], np.float32),
               prob=rng.random(m).astype(np.float32))
    for act, d in [("none", "bf16"), ("swiglu", "bf16"), ("srelu", "bf16")]:
        out = O.grouped_gemm(_problem(L, m, n, k, act=act, d=d, s=3.0), arr)
        grp = out["group"]
        for g in range(L):
            vals = [abs(v) for r in range(m) if grp[r] == g for v in out["d"][r]]
            assert out["amax"][g] == (max(vals) if vals else 0.0)


# ---------------------------------------------------------------------------
# P-e: SwiGLU closed forms
# ---------------------------------------------------------------------------

def test_swiglu_closed_forms(O):
    sig = lambda t: 1.0 / (1.0 + math.exp(-t))
    xs = [-3.0, -0.5, 0.0, 1.0, 2.5]
    gs = [-40.0, -2.0, 0.0, 0.7, 3.0, 40.0]
    for x, g in itertools.product(xs, gs):
        c = np.concatenate([np.full(32, x), np.full(32, g)])[None, :]
        d = O.swiglu(c, np.array([0.3]))
        assert np.allclose(d, 0.3 * x * g * sig(g), rtol=1e-15, atol=1e-300)
    # sigma(-t) = 1 - sigma(t): swish(g) - swish(-g) = g
    c1 = np.concatenate([np.ones(32), np.full(32, 1.7)])[None]
    c2 = np.concatenate([np.ones(32), np.full(32, -1.7)])[None]
    assert np.allclose(O.swiglu(c1, np.ones(1)) - O.swiglu(c2, np.ones(1)), 1.7, rtol=1e-15)
    # large gate: swish(g) -> g; very negative gate -> 0
    c = np.concatenate([np.full(32, 2.0), np.full(32, 60.0)])[None]
    assert np.allclose(O.swiglu(c, np.ones(1)), 120.0, rtol=1e-15)


def test_swiglu_pairs_independent(O):
    # changing pair b only changes output block b
    rng = np.random.default_rng(2)
    c = rng.standard_normal((3, 256))
    base = O.swiglu(c, np.ones(3))
    c2 = c.copy()
    c2[:, 128:192] += 1.0
    d2 = O.swiglu(c2, np.ones(3))
    changed = np.any(d2 != base, axis=0)
    assert not changed[:64].any() and changed[64:96].all() and not changed[96:].any()


# ---------------------------------------------------------------------------
# P-f: sReLU and the tanh soft clamp
# ---------------------------------------------------------------------------

def test_srelu_properties(O):
    rng = np.random.default_rng(4)
    c = rng.standard_normal((64, 128)) * 40
    p = rng.random(64)
    for s in [0.5, 8.0, 32.0]:
        d = O.srelu(c, p, s)
        assert np.all(d <= s * s * p[:, None] * (1 + 1e-15))
        assert np.all(d[c <= 0] == 0)
    d_plain = O.srelu(c, p, 0.0)
    assert np.array_equal(d_plain, p[:, None] * np.maximum(c, 0) ** 2)
    d_big = O.srelu(c, p, 1e8)          # (r/s)^2 <= 1e-11
    np.testing.assert_allclose(d_big, d_plain, rtol=1e-9)
    # small-r series: (s tanh(r/s))^2 = r^2 (1 - 2 r^2 / (3 s^2) + O(r^4/s^4))
    r = np.array([[1e-3, 1e-2, 0.05]])
    s = 8.0
    series = r ** 2 * (1 - 2 * r ** 2 / (3 * s * s))
    np.testing.assert_allclose(O.srelu(r, np.ones(1), s), series, rtol=1e-9)


# ---------------------------------------------------------------------------
# P-g: dSwiGLU and dprob by central finite differences of the forward
# ---------------------------------------------------------------------------

def test_dswiglu_matches_finite_differences(O):
    rng = np.random.default_rng(8)
    rows, n = 3, 64
    R = rng.standard_normal((rows, n))
    X = rng.standard_normal((rows, 2 * n)) * 2
    p = rng.random(rows)

    def loss(Xv, pv):
        # L = sum_j R[m,j] * f_j with f = p * input * swish(gate), pairs [input|gate]
        xs = Xv.reshape(rows, n // 32, 2, 32)
        inp, gate = xs[:, :, 0, :], xs[:, :, 1, :]
        f = pv[:, None, None] * inp * gate / (1 + np.exp(-gate))
        return (R.reshape(rows, n // 32, 32) * f).sum()

    dc, dprob = O.dswiglu(R, X, p)
    h = 1e-6
    num = np.zeros_like(X)
    for r in range(rows):
        for j in range(2 * n):
            Xp, Xm = X.copy(), X.copy()
            Xp[r, j] += h
            Xm[r, j] -= h
            num[r, j] = (loss(Xp, p) - loss(Xm, p)) / (2 * h)
    np.testing.assert_allclose(dc, num, rtol=1e-6, atol=1e-8)
    nump = np.zeros(rows)
    for r in range(rows):
        pp, pm = p.copy(), p.copy()
        pp[r] += h
        pm[r] -= h
        nump[r] = (loss(X, pp) - loss(X, pm)) / (2 * h)
    np.testing.assert_allclose(dprob, nump, rtol=1e-7, atol=1e-9)


def test_dswiglu_alpha_squared_and_beta_placement(O):
    m, k, n = 2, 32, 32
    arr = dict(a=np.full((m, k), 0x3F80, np.uint16), b=np.full((1, n, k), 0x3D00, np.uint16),
               padded_offsets=np.array([m], np.int32), alpha=np.array([3.0], np.float32),
               beta=np.array([0.25], np.float32), prob=np.array([1.0, 0.5], np.float32),
               c_in=np.full((m, 2 * n), 0x4000, np.uint16))          # 2.0 -> X = 0.5
    out = O.grouped_gemm(_problem(1, m, n, k, ab="bf16", act="dswiglu"), arr)
    assert np.all(out["r"] == 9.0)                                   # alpha^2 * (32 * 2^-5)
    s = 1 / (1 + math.exp(-0.5))
    np.testing.assert_allclose(out["dc"][0, :32], 9.0 * 0.5 * s, rtol=1e-15)
    np.testing.assert_allclose(out["dprob"], 32 * 9.0 * 0.5 * 0.5 * s, rtol=1e-14)


@pytest.mark.parametrize("s_clamp", [0.0, 2.0])
def test_dsrelu_matches_finite_differences(s_clamp, O):
    """dC and dprob of the sReLU backward against central differences of the
    forward loss L = sum R * prob * f(C), f from the sReLU page's equations."""
    rng = np.random.default_rng(9)
    rows, n = 3, 40
    R = rng.standard_normal((rows, n))
    C = rng.standard_normal((rows, n)) * 3
    C[np.abs(C) < 1e-3] = 0.5                     # keep away from the kink at 0
    p = rng.random(rows)

    def loss(Cv, pv):
        return (R * O.srelu(Cv, pv, s_clamp)).sum()

    dc, dprob = O.dsrelu(R, C, p, s_clamp)
    h = 1e-6
    num = np.zeros_like(C)
    for r in range(rows):
        for j in range(n):
            Cp, Cm = C.copy(), C.copy()
            Cp[r, j] += h
            Cm[r, j] -= h
            num[r, j] = (loss(Cp, p) - loss(Cm, p)) / (2 * h)
    np.testing.assert_allclose(dc, num, rtol=1e-6, atol=1e-8)
    nump = np.zeros(rows)
    for r in range(rows):
        pp, pm = p.copy(), p.copy()
        pp[r] += h
        pm[r] -= h
        nump[r] = (loss(C, pp) - loss(C, pm)) / (2 * h)
    np.testing.assert_allclose(dprob, nump, rtol=1e-7, atol=1e-9)
    assert np.all(dc[C <= 0] == 0.0)


def test_dsrelu_through_the_gemm_closed_form(O):
    """R = alpha^2 * acc, C read without scaling: A = 1.0 (byte 127), B = 1/32
    (byte 122), K = 64 -> acc = 2, alpha 0.5 -> R = 0.5; C = 2.0, s = 0:
    dC = 0.5 * prob * 4, dprob = 0.5 * 64 columns * 4 = 128 (N = 64)."""
    m, k, n = 2, 64, 64
    a, sfa = _const_mx(m, k, 0x38, 127)
    b, sfb = _const_mx(n, k, 0x38, 122)
    arr = dict(a=a, sfa=sfa, b=b.reshape(1, n, k), sfb=sfb.reshape(1, n, k // 32),
               padded_offsets=np.array([m], np.int32), alpha=np.array([0.5], np.float32),
               prob=np.array([1.0, 0.25], np.float32), c_in=np.full((m, n), 0x4000, np.uint16))
    out = O.grouped_gemm(_problem(1, m, n, k, ab="e4m3", act="dsrelu", d="bf16"), arr)
    np.testing.assert_array_equal(out["dc"], np.repeat([[2.0], [0.5]], n, axis=1))
    np.testing.assert_array_equal(out["dprob"], [128.0, 128.0])
    np.testing.assert_array_equal(out["amax"], [2.0])


def test_e5m2_is_the_upper_byte_of_binary16():
    """Every E5M2 code decodes to the IEEE binary16 value whose upper byte it
    is (numpy's float16 is the reference)."""
    c = np.arange(256)
    ref = (c.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    got = F.decode_e5m2(c)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert got[0x3C] == 1.0 and got[0x7B] == 57344.0 and got[0x01] == 2.0 ** -16 and got[0x7C] == np.inf


def test_dgeglu_matches_finite_differences_of_geglu(O):
    """Without clamps the dGeGLU backward is the derivative of the GeGLU forward:
    with L = sum R * D(C) over the GeGLU outputs, dC = dL/dC and dprob = dL/dprob
    (R indexed by output column, the pairs [gate | up] gate first)."""
    rng = np.random.default_rng(10)
    rows, nb = 3, 2                      # 2 pairs -> C width 128, output width 64
    R = rng.standard_normal((rows, 32 * nb))
    C = rng.standard_normal((rows, 64 * nb)) * 2
    p = rng.random(rows)
    a, off = 1.3, 0.75

    def loss(Cv, pv):
        return (R * O.geglu(Cv, pv, 1.0, a, off, -np.inf, np.inf)).sum()

    dc, dprob = O.dgeglu(R, C, p, a, off, -np.inf, np.inf)
    h = 1e-6
    num = np.zeros_like(C)
    for r in range(rows):
        for j in range(C.shape[1]):
            Cp, Cm = C.copy(), C.copy()
            Cp[r, j] += h
            Cm[r, j] -= h
            num[r, j] = (loss(Cp, p) - loss(Cm, p)) / (2 * h)
    np.testing.assert_allclose(dc, num, rtol=1e-6, atol=1e-8)
    nump = np.array([(loss(C, p + h * (np.arange(rows) == r)) - loss(C, p - h * (np.arange(rows) == r))) / (2 * h)
                     for r in range(rows)])
    np.testing.assert_allclose(dprob, nump, rtol=1e-7, atol=1e-9)


def test_dgeglu_clamp_masks_closed_form(O):
    """Gate above clamp_max: dgate = 0, dup uses the clamped gate; up outside
    [min, max]: dup = 0, dgate uses the clamped up; equality keeps the gradient."""
    R = np.ones((1, 32))
    c = np.zeros((1, 64))
    c[0, :32] = [9.0, 7.0, 1.0, 1.0] + [0.0] * 28          # gate
    c[0, 32:] = [2.0, 2.0, -9.0, 7.0] + [0.0] * 28         # up
    dc, dprob = O.dgeglu(R, c, np.ones(1), 1.702, 1.0, -7.0, 7.0)
    s7 = 1 / (1 + np.exp(-1.702 * 7.0))
    s1 = 1 / (1 + np.exp(-1.702))
    assert dc[0, 0] == 0.0                                  # gate 9 > 7
    np.testing.assert_allclose(dc[0, 32], 7.0 * s7, rtol=1e-15)            # dup with gate_c = 7
    np.testing.assert_allclose(dc[0, 1], 3.0 * s7 * (1 + 1.702 * 7 * (1 - s7)), rtol=1e-15)   # gate == 7 kept
    assert dc[0, 34] == 0.0                                 # up -9 < -7
    np.testing.assert_allclose(dc[0, 2], (-7.0 + 1.0) * s1 * (1 + 1.702 * (1 - s1)), rtol=1e-15)
    np.testing.assert_allclose(dc[0, 35], 1.0 * s1, rtol=1e-15)             # up == 7 kept
    np.testing.assert_allclose(dprob[0], 7 * s7 * 3 + 7 * s7 * 3 + s1 * (-6) + s1 * 8, rtol=1e-14)


def test_geglu_is_sigmoid_gelu_times_up(O):
    """GeGLU with offset 1, gamma 1 and no clamp: D = (U + 1) * G * sigmoid(1.702 G),
    checked against scipy's logistic function; the clamp bounds both halves."""
    from scipy.special import expit
    rng = np.random.default_rng(11)
    c = rng.standard_normal((4, 128)) * 3
    p = rng.random(4)
    d = O.geglu(c, p, 1.0, 1.702, 1.0, -np.inf, np.inf)
    g, u = c[:, :32], c[:, 32:64]
    np.testing.assert_allclose(d[:, :32], p[:, None] * (u + 1) * g * expit(1.702 * g), rtol=1e-13)
    dcl = O.geglu(c, p, 2.0, 1.702, 1.0, -1.0, 1.0)
    gc, uc = np.clip(g, -1, 1), np.clip(u, -1, 1)
    np.testing.assert_allclose(dcl[:, :32], 2 * p[:, None] * (uc + 1) * gc * expit(1.702 * gc), rtol=1e-13)


def _bs_dswiglu_case(d_dtype):
    """Two experts of 2 rows, MXFP8 A = 1.0 and B = 1/32 (scale byte 122), K = 64:
    acc = 2; alpha = (0.5, 1) -> R = (0.5, 2).  C_in: input blocks 2.0, gate
    blocks 0.0 (beta 1), so swish(gate) = 0 and sigmoid(gate) = 1/2:
    d_input = 0, d_gate = R * prob * 2 * 1/2 = R * prob, dprob = 0."""
    m, k, n = 4, 64, 32
    a, sfa = _const_mx(m, k, 0x38, 127)
    b, sfb = _const_mx(2 * n, k, 0x38, 122)
    c_in = np.zeros((m, 2 * n), np.uint16)
    c_in[:, :32] = 0x4000
    arr = dict(a=a, sfa=sfa, b=b.reshape(2, n, k), sfb=sfb.reshape(2, n, k // 32),
               padded_offsets=np.array([2, 4], np.int32), alpha=np.array([0.5, 1.0], np.float32),
               beta=np.ones(2, np.float32), prob=np.array([1.0, 0.5, 1.0, 0.25], np.float32),
               c_in=c_in, norm_const=np.ones(1, np.float32))
    return _problem(2, m, n, k, ab="e4m3", act="dswiglu", d=d_dtype), arr


def test_block_scaled_dswiglu_amax_pairs_closed_form(O):
    prob_, arr = _bs_dswiglu_case("bf16")
    out = O.grouped_gemm(prob_, arr)
    np.testing.assert_array_equal(out["r"], np.repeat([[0.5], [0.5], [2.0], [2.0]], 32, axis=1))
    assert np.all(out["dc"][:, :32] == 0.0)
    np.testing.assert_array_equal(out["dc"][:, 32], [0.5, 0.25, 2.0, 0.5])
    np.testing.assert_array_equal(out["dprob"], 0.0)
    # (L, 2): [max |d_input|, max |d_gate|] per expert
    np.testing.assert_array_equal(out["amax2"], [[0.0, 0.5], [0.0, 2.0]])


def test_block_scaled_dswiglu_fp8_dc_closed_form(O):
    prob_, arr = _bs_dswiglu_case("e4m3")
    out = O.grouped_gemm(prob_, arr)
    # input blocks all zero: byte 0, codes 0.  Gate block of row 0: amax 0.5,
    # smallest 2^e >= 0.5/448 is 2^-9 (byte 118), 0.5 / 2^-9 = 256 = E4M3 0x78;
    # row 1 (0.25): 2^-10 (byte 117), code 0x78 again
    np.testing.assert_array_equal(out["sfd_row"][:, 0], 0)
    np.testing.assert_array_equal(out["sfd_row"][:, 1], [118, 117, 120, 118])
    assert np.all(out["d_code"][:, :32] == 0) and np.all(out["d_code"][:, 32:] == 0x78)


# ---------------------------------------------------------------------------
# P-i: quantisation invariants
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nc", [1.0, 4.0, 0.125, 3.0])
def test_quantization_invariants(nc, O):
    rng = np.random.default_rng(6)
    d = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    d[5, 32:64] = 0.0                                                # an all-zero row block
    codes, sfd = O.quantize_rows(d, nc)
    d32 = d.astype(np.float32).astype(np.float64)
    blk = np.abs(d32).reshape(64, 8, 32).max(axis=2)
    scale = F.decode_e8m0(sfd)
    nz = blk > 0
    ratio = nc * blk[nz] / scale[nz]
    assert np.all(ratio > 224 * (1 - 1e-6)) and np.all(ratio <= 448 * (1 + 1e-6))
    assert sfd[5, 1] == 0 and np.all(codes[5, 32:64] == 0)
    vals = F.decode_e4m3(codes)
    assert np.all(np.abs(vals) <= 448)
    # dequantised value within half an E4M3 ULP of D*nc/SFD
    scaled = d32 * nc / np.repeat(scale, 32, axis=1)
    ex = np.floor(np.log2(np.maximum(np.abs(scaled), 2.0 ** -6)))
    half_ulp = 2.0 ** (ex - 3) / 2
    assert np.all(np.abs(vals - scaled) <= half_ulp * (1 + 1e-6) + 1e-30)
    # columns: same invariants on 32-row blocks
    ccodes, csfd = O.quantize_cols(d, nc)
    assert csfd.shape == (256, 2)
    cblk = np.abs(d32).reshape(2, 32, 256).max(axis=1).T
    cscale = F.decode_e8m0(csfd)
    nzc = cblk > 0
    r2 = nc * cblk[nzc] / cscale[nzc]
    assert np.all(r2 > 224 * (1 - 1e-6)) and np.all(r2 <= 448 * (1 + 1e-6))


def test_scale_exact_power_of_two_keeps_exponent(O):
    # amax * rcp_max exactly 2^-3 in float32 -> byte 124 (no round-up past it)
    amax = np.float32(2.0 ** -3) / RCP_MAX_E4M3
    sf = np.float32(amax) * RCP_MAX_E4M3
    byte = O.e8m0_block_scale(np.array([amax], np.float32), 1.0)[0]
    m, e = math.frexp(float(sf))
    assert byte == (e - 1 if m == 0.5 else e) + 127


# ---------------------------------------------------------------------------
# hand-worked examples (tests/golden/worked_examples.yaml)
# ---------------------------------------------------------------------------

def _build(case):
    p = dict(case["problem"])
    p.setdefault("c_dtype", None)
    p.setdefault("srelu_tanh_s", 0.0)
    m, n, k, L = p["valid_m"], p["n"], p["k"], p["num_groups"]
    ab = p["ab_dtype"]
    fp4 = ab == "e2m1x2"
    kb = k // 2 if fp4 else k
    arr = dict(padded_offsets=np.array(case["po"], np.int32),
               alpha=np.array(case["alpha"], np.float32),
               norm_const=np.array([case.get("norm_const", 1.0)], np.float32))
    if "prob" in case:
        arr["prob"] = np.array(case["prob"], np.float32)
    else:
        arr["prob"] = np.full(m, case["prob_const"], np.float32)
    if ab == "bf16":
        arr["a"] = np.zeros((m, k), np.uint16)
        for r, bits in enumerate(case["a_bf16_rows"]):
            arr["a"][r] = bits
        arr["b"] = np.zeros((L, n, k), np.uint16)
        for g, r0, r1, bits in case["b_bf16_rows"]:
            arr["b"][g, r0:r1] = bits
        arr["beta"] = np.array(case["beta"], np.float32)
        arr["c_in"] = np.zeros((m, 2 * n), np.uint16)
        for c0, c1, bits in case["c_in_blocks"]:
            arr["c_in"][:, c0:c1] = bits
    else:
        arr["a"] = np.zeros((m, kb), np.uint8)
        arr["sfa"] = np.zeros((m, k // 32), np.uint8)
        if "a_rows" in case:
            for r, (code, byte) in enumerate(case["a_rows"]):
                arr["a"][r], arr["sfa"][r] = code, byte
        else:
            code, byte0, period = case["a_rows_pattern"]
            for r in range(m):
                arr["a"][r], arr["sfa"][r] = code, byte0 + r % period
        arr["b"] = np.zeros((L, n, kb), np.uint8)
        arr["sfb"] = np.zeros((L, n, k // 32), np.uint8)
        for g, r0, r1, code, byte in case["b_blocks"]:
            arr["b"][g, r0:r1], arr["sfb"][g, r0:r1] = code, byte
    return p, arr


with open(GOLDEN) as _f:
    _CASES = yaml.safe_load(_f)


@pytest.mark.parametrize("case", _CASES, ids=[c["name"] for c in _CASES])
def test_worked_example(case, O):
    p, arr = _build(case)
    out = O.grouped_gemm(p, arr)
    ev = lambda s: eval(s, {"math": math})
    if "expect_d" in case:
        for r, v in enumerate(case["expect_d"]):
            assert np.all(out["d"][r] == v)
    if "expect_d_expr" in case:
        for r, s in enumerate(case["expect_d_expr"]):
            np.testing.assert_allclose(out["d"][r], ev(s), rtol=1e-14)
    for key in ("expect_d_cols", "expect_d_cols_expr", "expect_dc_cols_expr"):
        for c0, c1, v in case.get(key, []):
            tgt = out["dc"] if key.startswith("expect_dc") else out["d"]
            val = ev(v) if isinstance(v, str) else v
            np.testing.assert_allclose(tgt[:, c0:c1], val, rtol=1e-14, atol=0)
    if "expect_dprob_expr" in case:
        np.testing.assert_allclose(out["dprob"], [ev(s) for s in case["expect_dprob_expr"]], rtol=1e-14)
    if "expect_d_bits" in case:
        for r, v in enumerate(case["expect_d_bits"]):
            assert np.all(out["d_bits"][r] == v)
    if "expect_amax" in case:
        assert list(out["amax"]) == case["expect_amax"]
    if "expect_sfd_row" in case:
        for r, v in enumerate(case["expect_sfd_row"]):
            assert np.all(out["sfd_row"][r] == v)
    if "expect_d_code" in case:
        for r, v in enumerate(case["expect_d_code"]):
            assert np.all(out["d_code"][r] == v)
    if "expect_sfd_row_pattern" in case:
        pat = case["expect_sfd_row_pattern"]
        for r in range(p["valid_m"]):
            assert np.all(out["sfd_row"][r] == pat[r % len(pat)])
    if "expect_d_code_const" in case:
        assert np.all(out["d_code"] == case["expect_d_code_const"])
    if "expect_sfd_col_const" in case:
        assert np.all(out["sfd_col"] == case["expect_sfd_col_const"])
    if "expect_d_col_code_pattern" in case:
        pat = case["expect_d_col_code_pattern"]
        for r in range(p["valid_m"]):
            assert np.all(out["d_col_code"][r] == pat[r % len(pat)])


# ---------------------------------------------------------------------------
# a planted mistake in the oracle must be caught by the pins above
# ---------------------------------------------------------------------------

def test_planted_block_order_swap_is_detected(monkeypatch):
    case = next(c for c in _CASES if c["name"] == "W2_swiglu_order")
    p, arr = _build(case)

    def swapped(c, prob):
        r, n = c.shape
        pairs = c.reshape(r, n // 64, 2, 32)
        g, x = pairs[:, :, 0, :], pairs[:, :, 1, :]          # wrong order
        return (prob[:, None, None] * x * (g * G.sigmoid(g))).reshape(r, n // 2)
    monkeypatch.setattr(G, "swiglu", swapped)
    out = oracle.grouped_gemm(p, arr)
    assert not np.allclose(out["d"][0], 1 / (1 + math.exp(-2)))


def test_dsrelu_derivative_in_the_saturated_clamp(O):
    """Far into the tanh clamp (relu(C)/s up to 300) the sReLU derivative's
    factor 1 - tanh^2 = sech^2 must keep its value: checked against
    4 e^-2x / (1 + e^-2x)^2, a form free of cancellation (an evaluation as
    1 - t*t is 0 or all rounding error once t rounds to 1, x > ~19)."""
    s = 0.5
    x = np.array([0.01, 0.2, 3.0, 9.0, 15.0, 19.5, 30.0, 150.0])
    c_saved = (x * s)[None, :]
    R = np.ones_like(c_saved)
    p = np.ones(1)
    dc, _ = O.dsrelu(R, c_saved, p, s)
    e = np.exp(-2.0 * x)
    t = (1.0 - e) / (1.0 + e)
    expect = 2.0 * s * t * 4.0 * e / (1.0 + e) ** 2
    np.testing.assert_allclose(dc[0], expect, rtol=1e-12, atol=0)
    assert dc[0, -1] > 0                                 # 4 e^-300: still a normal float64
