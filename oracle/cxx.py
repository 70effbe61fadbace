"""ctypes binding of the C++ oracle (``oracle/cpp``), with the numpy oracle's
function names and return layout.

TEST INFRASTRUCTURE ONLY.  See ``oracle/__init__.py``.  Argument marshalling
only: every step of the computation is in ``oracle/cpp/oracle.cpp``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "cpp")
LIB_PATH = os.path.join(HERE, "liboracle.so")
SOURCES = [os.path.join(HERE, "oracle.cpp")]

E4M3, E5M2, E2M1, BF16, E8M0 = 0, 1, 2, 3, 4
_AB = {"e4m3": E4M3, "e5m2": E5M2, "e2m1x2": E2M1, "bf16": BF16}
_ACT = {"none": 0, "swiglu": 1, "srelu": 2, "dswiglu": 3, "dsrelu": 4, "geglu": 5, "dgeglu": 6}


def build() -> str:
    """Compile the oracle with g++ (plain IEEE arithmetic: no fast-math, no
    contraction of multiplies and adds), OpenMP over rows."""
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", *SOURCES]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("building the C++ oracle failed:\n" + r.stderr[-4000:])
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Problem(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("valid_m", ctypes.c_int64), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("ab", ctypes.c_int32), ("act", ctypes.c_int32), ("d_fp8", ctypes.c_int32),
                ("c_out", ctypes.c_int32), ("srelu_s", ctypes.c_double), ("glu_gamma", ctypes.c_double),
                ("geglu_alpha", ctypes.c_double), ("linear_offset", ctypes.c_double),
                ("clamp_min", ctypes.c_double), ("clamp_max", ctypes.c_double), ("norm_const", ctypes.c_float)]


class _Inputs(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in ("a", "sfa", "b", "sfb", "padded_offsets", "alpha", "beta", "prob",
                                               "c_in")]


class _Outputs(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in ("group", "cr", "d", "dprob", "c_bits", "d_bits", "d_code", "sfd_row",
                                               "d_col_code", "sfd_col", "amax")]


_lib = None


def lib():
    """The loaded library; built first if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I, O = ctypes.POINTER(_Problem), ctypes.POINTER(_Inputs), ctypes.POINTER(_Outputs)
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.ox_run.argtypes, L.ox_run.restype = [P, I, vp, i64, O], ctypes.c_int
        L.ox_threads.restype = ctypes.c_int
        L.ox_last_error.restype = ctypes.c_char_p
        L.ox_decode.argtypes = [ctypes.c_int, vp, i64, vp]
        L.ox_decode_bf16.argtypes = [vp, i64, vp]
        L.ox_encode_e4m3.argtypes = [vp, i64, vp]
        L.ox_encode_bf16.argtypes = [vp, i64, vp]
        L.ox_e8m0_scale.argtypes, L.ox_e8m0_scale.restype = [ctypes.c_float, ctypes.c_float], ctypes.c_uint8
        L.ox_activation.argtypes, L.ox_activation.restype = [P, i64, vp, vp, vp, vp, vp], ctypes.c_int
        L.ox_quantize.argtypes, L.ox_quantize.restype = [ctypes.c_int, vp, i64, i64, ctypes.c_float, vp, vp], ctypes.c_int
        _lib = L
    return _lib


def threads() -> int:
    return int(lib().ox_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc:
        raise ValueError("C++ oracle: " + lib().ox_last_error().decode())


def _c(a, dtype):
    return np.array(a, dtype=dtype, order="C")          # a C-ordered copy (0-d stays 0-d)


def _problem(problem: dict) -> _Problem:
    p = _Problem()
    p.num_groups, p.valid_m = int(problem["num_groups"]), int(problem["valid_m"])
    p.n, p.k = int(problem["n"]), int(problem["k"])
    p.ab, p.act = _AB[problem["ab_dtype"]], _ACT[problem["act"]]
    p.d_fp8 = 1 if problem.get("d_dtype") == "e4m3" else 0
    p.c_out = 1 if problem.get("c_dtype") == "bf16" else 0
    p.srelu_s = float(problem.get("srelu_tanh_s", 0.0))
    p.glu_gamma = float(problem.get("glu_gamma", 1.0))
    p.geglu_alpha = float(problem.get("geglu_alpha", 1.702))
    p.linear_offset = float(problem.get("linear_offset", 1.0))
    p.clamp_min = float(problem.get("glu_clamp_min", -np.inf))
    p.clamp_max = float(problem.get("glu_clamp_max", np.inf))
    p.norm_const = 1.0
    return p


def n_out(problem: dict) -> int:
    n, act = int(problem["n"]), problem["act"]
    return {"swiglu": n // 2, "geglu": n // 2, "dswiglu": 2 * n, "dgeglu": 2 * n}.get(act, n)


# ---------------------------------------------------------------------------
# the whole path
# ---------------------------------------------------------------------------

def grouped_gemm(problem: dict, arrays: dict, rows=None) -> dict:
    """The C++ oracle over the given rows (default: all), returned under the
    numpy oracle's keys: 'rows', 'group', 'c' or 'r', 'd' or 'dc' (+ 'dprob',
    'dc_bits'), 'c_bits', 'd_bits' + 'amax' / 'amax2', or 'd_code', 'sfd_row'
    and, for whole aligned 32-row blocks, 'd_col_code', 'sfd_col', 'col_blocks'."""
    p = _problem(problem)
    nc = arrays.get("norm_const")
    if nc is not None:
        p.norm_const = float(np.asarray(nc, np.float32).reshape(-1)[0])
    valid_m, n, L = p.valid_m, p.n, p.num_groups
    rows = np.arange(valid_m, dtype=np.int64) if rows is None else _c(rows, np.int64).reshape(-1)
    m, no, act = len(rows), n_out(problem), problem["act"]
    bwd, mx = act in ("dswiglu", "dsrelu", "dgeglu"), problem["ab_dtype"] != "bf16"
    fp8 = p.d_fp8 == 1

    keep = []

    def inp(key, dtype):
        a = arrays.get(key)
        if a is None:
            return None
        a = _c(a, dtype)
        keep.append(a)
        return _ptr(a)
    code_t = np.uint16 if problem["ab_dtype"] == "bf16" else np.uint8
    ins = _Inputs(a=inp("a", code_t), sfa=inp("sfa", np.uint8), b=inp("b", code_t), sfb=inp("sfb", np.uint8),
                  padded_offsets=inp("padded_offsets", np.int32), alpha=inp("alpha", np.float32),
                  beta=inp("beta", np.float32), prob=inp("prob", np.float32), c_in=inp("c_in", np.uint16))
    o = {"group": np.zeros(m, np.int32), "cr": np.zeros((m, n)), "d": np.zeros((m, no)),
         "dprob": np.zeros(m), "d_bits": np.zeros((m, no), np.uint16)}
    if problem.get("c_dtype") == "bf16" and not bwd:
        o["c_bits"] = np.zeros((m, n), np.uint16)
    if fp8 and (mx or not bwd):
        o.update(d_code=np.zeros((m, no), np.uint8), sfd_row=np.zeros((m, no // 32), np.uint8),
                 d_col_code=np.zeros((m, no), np.uint8), sfd_col=np.zeros((no, max(m // 32, 1)), np.uint8))
    pairs = act in ("dswiglu", "dgeglu") and mx and not fp8
    if not fp8 and (mx or not bwd):
        o["amax"] = np.zeros((L, 2) if pairs else L)
    outs = _Outputs(**{f: _ptr(o.get(f)) for f, _ in _Outputs._fields_})
    _check(lib().ox_run(ctypes.byref(p), ctypes.byref(ins), _ptr(rows), m, ctypes.byref(outs)))

    res = {"rows": rows, "group": o["group"].astype(np.int64)}
    if bwd:
        res.update(r=o["cr"], dc=o["d"], dprob=o["dprob"], dc_bits=o["d_bits"])
        if not mx:
            return res
        if pairs:
            res["amax2"] = o["amax"]
            return res
        res["d"] = o["d"]
    else:
        res.update(c=o["cr"], d=o["d"])
        if "c_bits" in o:
            res["c_bits"] = o["c_bits"]
    if not fp8:
        res.update(d_bits=o["d_bits"], amax=o["amax"])
        return res
    res.update(d_code=o["d_code"], sfd_row=o["sfd_row"])
    whole = (m % 32 == 0 and m > 0 and np.all(rows.reshape(-1, 32) == rows.reshape(-1, 32)[:, :1] + np.arange(32))
             and np.all(rows.reshape(-1, 32)[:, 0] % 32 == 0))
    if whole:
        res.update(d_col_code=o["d_col_code"], sfd_col=o["sfd_col"], col_blocks=rows.reshape(-1, 32)[:, 0] // 32)
    return res


# ---------------------------------------------------------------------------
# the steps on their own (the pins call these)
# ---------------------------------------------------------------------------

def _decode(fmt, codes):
    c = _c(codes, np.uint8)
    out = np.zeros(c.shape)
    lib().ox_decode(fmt, _ptr(c), c.size, _ptr(out))
    return out


def decode_e4m3(codes):
    return _decode(E4M3, codes)


def decode_e5m2(codes):
    return _decode(E5M2, codes)


def decode_e2m1(nibbles):
    return _decode(E2M1, nibbles)


def decode_e8m0(codes):
    return _decode(E8M0, codes)


def decode_bf16(bits):
    b = _c(bits, np.uint16)
    out = np.zeros(b.shape)
    lib().ox_decode_bf16(_ptr(b), b.size, _ptr(out))
    return out


def encode_e4m3(values):
    v = _c(values, np.float64)
    out = np.zeros(v.shape, np.uint8)
    lib().ox_encode_e4m3(_ptr(v), v.size, _ptr(out))
    return out


def encode_bf16(values):
    v = _c(values, np.float64)
    out = np.zeros(v.shape, np.uint16)
    lib().ox_encode_bf16(_ptr(v), v.size, _ptr(out))
    return out


def e8m0_block_scale(amax32, nc32):
    a = np.asarray(amax32, np.float32)
    return np.array([lib().ox_e8m0_scale(float(x), float(np.float32(nc32))) for x in a.reshape(-1)],
                    np.uint8).reshape(a.shape)


def _act(problem, cr, prob, saved=None):
    p = _problem(problem)
    cr, prob = _c(cr, np.float64), _c(prob, np.float64)
    rows = cr.shape[0]
    d = np.zeros((rows, n_out(problem)))
    dprob = np.zeros(rows)
    sv = None if saved is None else _c(saved, np.float64)
    _check(lib().ox_activation(ctypes.byref(p), rows, _ptr(cr), _ptr(prob), _ptr(sv), _ptr(d), _ptr(dprob)))
    return d, dprob


def _shape(act, n, **kw):
    return dict(num_groups=1, valid_m=0, n=n, k=32, ab_dtype="e4m3", act=act, d_dtype="bf16", **kw)


def swiglu(c, prob):
    return _act(_shape("swiglu", np.shape(c)[1]), c, prob)[0]


def srelu(c, prob, s: float):
    return _act(_shape("srelu", np.shape(c)[1], srelu_tanh_s=float(s)), c, prob)[0]


def geglu(c, prob, gamma, alpha, offset, cmin, cmax):
    kw = dict(glu_gamma=gamma, geglu_alpha=alpha, linear_offset=offset, glu_clamp_min=cmin, glu_clamp_max=cmax)
    return _act(_shape("geglu", np.shape(c)[1], **kw), c, prob)[0]


def dswiglu(rmat, x_saved, prob):
    return _act(_shape("dswiglu", np.shape(rmat)[1]), rmat, prob, x_saved)


def dsrelu(rmat, c_saved, prob, s: float):
    return _act(_shape("dsrelu", np.shape(rmat)[1], srelu_tanh_s=float(s)), rmat, prob, c_saved)


def dgeglu(rmat, c_saved, prob, alpha, offset, cmin, cmax):
    kw = dict(geglu_alpha=alpha, linear_offset=offset, glu_clamp_min=cmin, glu_clamp_max=cmax)
    return _act(_shape("dgeglu", np.shape(rmat)[1], **kw), rmat, prob, c_saved)


def _quant(axis, d64, nc):
    d = _c(d64, np.float64)
    r, n = d.shape
    codes = np.zeros((r, n), np.uint8)
    sf = np.zeros((r, n // 32) if axis == 0 else (n, r // 32), np.uint8)
    _check(lib().ox_quantize(axis, _ptr(d), r, n, float(np.float32(nc)), _ptr(codes), _ptr(sf)))
    return codes, sf


def quantize_rows(d64, nc: float):
    return _quant(0, d64, nc)


def quantize_cols(d64, nc: float):
    return _quant(1, d64, nc)
