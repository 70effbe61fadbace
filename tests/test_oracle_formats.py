"""Pins of the oracles' format codecs against library routines and the format
tables (tests/golden/format_values.txt).  Every pin runs on the numpy oracle's
codecs (``oracle.formats``) and on the C++ oracle's (``oracle/cpp`` through
``oracle.cxx``).  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as NF


@pytest.fixture(params=["numpy", "cpp"])
def F(request):
    """Each pin runs against both oracles' codecs."""
    if request.param == "numpy":
        return NF
    from oracle import cxx
    return cxx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "format_values.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        rows.append(line.split())
    return rows


def _eq_or_both_nan(a, b):
    return (math.isnan(a) and math.isnan(b)) or a == b


def test_golden_landmarks(F):
    for fmt, code, val in _golden_rows():
        if fmt == "qmax":
            if code == "e4m3":
                assert NF.E4M3_MAX == float(val)
                assert F.decode_e4m3(0x7E) == float(val)
            continue
        c = int(code, 16)
        got = {"e4m3": F.decode_e4m3, "e2m1": F.decode_e2m1, "e8m0": F.decode_e8m0}[fmt](c)
        assert _eq_or_both_nan(float(got), float(val)), (fmt, code, got, val)


def test_e4m3_decode_all_codes_vs_torch(F):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.decode_e4m3(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e8m0_decode_all_codes_vs_torch(F):
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = F.decode_e8m0(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e2m1_table_and_unpack_order(F):
    vals = F.decode_e2m1(np.arange(16))
    assert list(vals[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(-vals[9:]) == [0.5, 1, 1.5, 2, 3, 4, 6]
    # low nibble is the even (first) K element (the C++ oracle unpacks inside
    # its GEMM; the FP4 brute-force pin covers its order)
    if F is NF:
        assert list(F.unpack_e2m1x2(np.array([[0x71]], np.uint8))[0]) == [1, 7]


def test_bf16_decode_vs_torch(F):
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.decode_bf16(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_e4m3_encode_roundtrip_every_finite_code(F):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and c != 0x80], np.uint8)
    assert np.array_equal(F.encode_e4m3(F.decode_e4m3(codes)), codes)


def test_e4m3_encode_vs_torch_random_and_midpoints(F):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200000) * 50,
        rng.uniform(-2 ** -6, 2 ** -6, 50000),            # subnormal range
        rng.uniform(-448, 448, 50000),
    ]).astype(np.float32)
    pos = F.decode_e4m3(np.arange(0x7F))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # every tie (exact in fp32)
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.encode_e4m3(x)
    # torch keeps the sign of a value that rounds to zero; the oracle emits +0
    ref = np.where((ref & 0x7F) == 0, 0, ref)
    assert np.array_equal(ref, got)


def test_e4m3_ties_go_to_even(F):
    pos = F.decode_e4m3(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    codes = F.encode_e4m3(mids)
    assert np.all(codes % 2 == 0)
    assert np.all((codes == np.arange(0x7E)) | (codes == np.arange(1, 0x7F)))


def test_e4m3_satfinite(F):
    big = np.array([448.0, 449.0, 464.0, 465.0, 1e6, 3e38, -1e6], np.float64)
    assert list(F.encode_e4m3(big)) == [0x7E] * 6 + [0xFE]


def test_bf16_encode_vs_torch(F):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(300000) * np.exp(rng.uniform(-20, 20, 300000))).astype(np.float32)
    # exact ties: low 16 bits = 0x8000 with both parities of the kept LSB
    tb = (rng.integers(0x0080, 0x7F00, 20000, dtype=np.uint32) << 16) | 0x8000
    x = np.concatenate([x, tb.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = F.encode_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_encode_rounds_fp64_once(F):
    # 1 + 2^-8 + 2^-30 is above the tie between 1 and 1+2^-7: must round up,
    # which a float32 detour (that drops 2^-30) would get wrong.
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert F.encode_bf16(np.array([v]))[0] == 0x3F81
    assert F.encode_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80


def test_e5m2_decode_is_the_upper_byte_of_binary16(F):
    """Every E5M2 code decodes to the IEEE binary16 value whose upper byte it
    is (numpy's float16 is the reference)."""
    c = np.arange(256)
    ref = (c.astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    got = F.decode_e5m2(c)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
