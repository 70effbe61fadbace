"""Python binding of libmoegg (ctypes).  Argument marshalling only.

The C ABI (include/moegg.h) is mirrored name for name:

    moegg_check(problem, args) -> status
    moegg_run(problem, args, stream) -> status
    moegg_check_offsets(problem, padded_offsets_ptr, stream) -> status
    moegg_n_out(problem), moegg_status_string(status), moegg_last_error(),
    moegg_abi_version(), moegg_set_grid_limit(max_workgroups),
    moegg_sf_to_kplanes(src, dst, rows, k, stream)

plus ``make_problem`` / ``make_args`` (fill the C structs from a problem dict
and torch tensors' device pointers) and ``run`` / ``check`` (build the structs,
call, raise ``MoeggError`` on a non-OK status).  Every step of the computation
runs in the HIP library; this module never computes.  If ``libmoegg.so`` has
not been built the first call raises ``RuntimeError``: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["MoeggError", "moegg_check", "moegg_run", "moegg_check_offsets", "moegg_n_out",
           "moegg_status_string", "moegg_last_error", "moegg_abi_version", "moegg_set_grid_limit", "make_problem",
           "make_args", "run", "check", "lib_path", "ABI_VERSION", "DTYPES", "ACTS", "STATUS", "SF_LAYOUTS",
           "moegg_sf_to_kplanes", "sf_to_kplanes"]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libmoegg.so")

ABI_VERSION = 5   # MOEGG_ABI_VERSION of the structs below
DTYPES = {None: 0, "none": 0, "e4m3": 1, "e2m1x2": 2, "bf16": 3, "e5m2": 4}
ACTS = {"none": 0, "swiglu": 1, "srelu": 2, "dswiglu": 3, "dsrelu": 4, "geglu": 5, "dgeglu": 6}
SF_LAYOUTS = {"row_major": 0, "kplanes": 1}
STATUS = {0: "MOEGG_OK", 1: "MOEGG_ERROR_INVALID_VALUE", 2: "MOEGG_ERROR_MISALIGNED",
          3: "MOEGG_ERROR_NOT_SUPPORTED", 4: "MOEGG_ERROR_LAUNCH"}

ARG_FIELDS = ("a", "b", "sfa", "sfb", "padded_offsets", "alpha", "prob", "beta", "norm_const",
              "c_in", "c", "d", "d_col", "sfd_row", "sfd_col", "amax", "dprob", "b_ptrs", "sfb_ptrs")


class moegg_problem(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("m_aligned", ctypes.c_int32),
                ("valid_m", ctypes.c_int64), ("n", ctypes.c_int32), ("k", ctypes.c_int32),
                ("ab_dtype", ctypes.c_int32), ("c_dtype", ctypes.c_int32),
                ("d_dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("srelu_tanh_s", ctypes.c_float), ("glu_gamma", ctypes.c_float),
                ("geglu_alpha", ctypes.c_float), ("linear_offset", ctypes.c_float),
                ("glu_clamp_min", ctypes.c_float), ("glu_clamp_max", ctypes.c_float),
                ("sf_layout", ctypes.c_int32)]


class moegg_args(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in ARG_FIELDS]


class MoeggError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built; run __graft_entry__.build() "
                               "(there is no fallback path)")
        lib = ctypes.CDLL(lib_path)
        P, A = ctypes.POINTER(moegg_problem), ctypes.POINTER(moegg_args)
        lib.moegg_check.argtypes, lib.moegg_check.restype = [P, A], ctypes.c_int
        lib.moegg_run.argtypes, lib.moegg_run.restype = [P, A, ctypes.c_void_p], ctypes.c_int
        lib.moegg_check_offsets.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p]
        lib.moegg_check_offsets.restype = ctypes.c_int
        lib.moegg_n_out.argtypes, lib.moegg_n_out.restype = [P], ctypes.c_int64
        lib.moegg_status_string.argtypes, lib.moegg_status_string.restype = [ctypes.c_int], ctypes.c_char_p
        lib.moegg_last_error.argtypes, lib.moegg_last_error.restype = [], ctypes.c_char_p
        lib.moegg_abi_version.argtypes, lib.moegg_abi_version.restype = [], ctypes.c_int
        lib.moegg_set_grid_limit.argtypes, lib.moegg_set_grid_limit.restype = [ctypes.c_int], ctypes.c_int
        lib.moegg_sf_to_kplanes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                            ctypes.c_void_p]
        lib.moegg_sf_to_kplanes.restype = ctypes.c_int
        if lib.moegg_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{lib_path} has ABI {lib.moegg_abi_version()}, these bindings "
                               f"expect {ABI_VERSION}: rebuild it with __graft_entry__.build()")
        _lib = lib
    return _lib


# ---- the C functions, same names ----------------------------------------------

def moegg_check(problem: moegg_problem, args: moegg_args) -> int:
    return _load().moegg_check(ctypes.byref(problem), ctypes.byref(args))


def moegg_run(problem: moegg_problem, args: moegg_args, stream: int | None) -> int:
    return _load().moegg_run(ctypes.byref(problem), ctypes.byref(args), stream or None)


def moegg_check_offsets(problem: moegg_problem, padded_offsets_ptr: int, stream: int | None) -> int:
    return _load().moegg_check_offsets(ctypes.byref(problem), padded_offsets_ptr, stream or None)


def moegg_n_out(problem: moegg_problem) -> int:
    return _load().moegg_n_out(ctypes.byref(problem))


def moegg_status_string(status: int) -> str:
    return _load().moegg_status_string(status).decode()


def moegg_last_error() -> str:
    return _load().moegg_last_error().decode()


def moegg_abi_version() -> int:
    return _load().moegg_abi_version()


def moegg_set_grid_limit(max_workgroups: int) -> int:
    return _load().moegg_set_grid_limit(int(max_workgroups))


def moegg_sf_to_kplanes(src_ptr: int, dst_ptr: int, rows: int, k: int, stream: int | None) -> int:
    return _load().moegg_sf_to_kplanes(src_ptr, dst_ptr, int(rows), int(k), stream or None)


# ---- marshalling helpers ---------------------------------------------------------

def _code(table: dict, v) -> int:
    return v if isinstance(v, int) else table[v]


def make_problem(p: dict) -> moegg_problem:
    """Problem dict (keys as in the C struct; dtypes/act as names or raw enum
    values) -> struct."""
    return moegg_problem(num_groups=int(p["num_groups"]), m_aligned=int(p.get("m_aligned", 128)),
                         valid_m=int(p["valid_m"]), n=int(p["n"]), k=int(p["k"]),
                         ab_dtype=_code(DTYPES, p["ab_dtype"]), c_dtype=_code(DTYPES, p.get("c_dtype")),
                         d_dtype=_code(DTYPES, p["d_dtype"]), act=_code(ACTS, p["act"]),
                         srelu_tanh_s=float(p.get("srelu_tanh_s", 0.0) or 0.0),
                         glu_gamma=float(p.get("glu_gamma", 1.0)),
                         geglu_alpha=float(p.get("geglu_alpha", 1.702)),
                         linear_offset=float(p.get("linear_offset", 1.0)),
                         glu_clamp_min=float(p.get("glu_clamp_min", float("-inf"))),
                         glu_clamp_max=float(p.get("glu_clamp_max", float("inf"))),
                         sf_layout=_code(SF_LAYOUTS, p.get("sf_layout", 0)))


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def make_args(tensors: dict) -> moegg_args:
    """Dict of torch tensors (or raw integer device pointers) -> struct of pointers."""
    unknown = set(tensors) - set(ARG_FIELDS)
    if unknown:
        raise KeyError(f"unknown tensor names {sorted(unknown)}")
    return moegg_args(**{k: _ptr(tensors.get(k)) for k in ARG_FIELDS})


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def check(problem: dict, tensors: dict) -> None:
    st = moegg_check(make_problem(problem), make_args(tensors))
    if st != 0:
        raise MoeggError(st, moegg_last_error())


def sf_to_kplanes(src, dst, rows: int, k: int, stream=None) -> None:
    """Enqueue the row-major -> K-block-plane scale conversion (device tensors or pointers)."""
    st = moegg_sf_to_kplanes(_ptr(src), _ptr(dst), rows, k, _stream_handle(stream))
    if st != 0:
        raise MoeggError(st, moegg_last_error())


def run(problem: dict, tensors: dict, stream=None) -> None:
    """Enqueue the grouped GEMM + epilogue on `stream` (default: torch's current)."""
    st = moegg_run(make_problem(problem), make_args(tensors), _stream_handle(stream))
    if st != 0:
        raise MoeggError(st, moegg_last_error())
