"""The parity rules themselves (CPU): rule 2's accounting of scale bytes that
pass only under the FP32-accumulation allowance, and its cap.

A planted device result is built from the oracle's own quantiser with one
block's scale byte lowered by one: the block's norm_const * amax / 448 sits
1e-4 above a power of two, outside rule 2's 1e-5 window, so only an
accumulation bound of 1e-3 on that block lets it pass, and it must then be
counted; two such blocks exceed the cap of a 64-block tensor."""
import numpy as np
import pytest

from oracle import formats as F
from oracle import grouped as G
from parity_util import rule2


def _planted(n_bad):
    rng = np.random.default_rng(11)
    rows, cols = 64, 32                   # 64 row blocks of 32 columns
    d = rng.uniform(-1.0, 1.0, (rows, cols))
    # rows 0 .. n_bad-1: block amax = 448 * 2^-3 * (1 + 1e-4)
    for r in range(n_bad):
        d[r, 5] = 448.0 * 2.0 ** -3 * (1.0 + 1e-4)
    codes, sf = G.quantize_rows(d, 1.0)
    sf = sf.copy()
    codes = codes.copy()
    for r in range(n_bad):
        assert sf[r, 0] == 127 - 3 + 1    # the exact amax rounds the scale up
        sf[r, 0] -= 1                     # the device's amax fell on the power of two
        codes[r] = F.encode_e4m3(np.clip(d[r] * 2.0 ** 3, -448.0, 448.0))
    bound = np.zeros_like(d)
    bound[:n_bad] = 1e-3                  # accumulation bound on the planted rows
    return d, codes, sf, bound


def test_widened_block_is_counted():
    d, codes, sf, bound = _planted(1)
    st = rule2(codes, sf, d, 1.0, "row", "planted", bound)
    assert st["scale_acc_allowance"] == 1
    assert st["scale_blocks"] == 64


def test_without_bound_the_block_fails():
    d, codes, sf, _ = _planted(1)
    with pytest.raises(AssertionError, match="away from a power-of-two boundary"):
        rule2(codes, sf, d, 1.0, "row", "planted")


def test_widened_blocks_above_cap_fail():
    d, codes, sf, bound = _planted(2)
    with pytest.raises(AssertionError, match="accumulation allowance"):
        rule2(codes, sf, d, 1.0, "row", "planted", bound)


def test_exact_result_counts_nothing():
    d, _, _, bound = _planted(0)
    codes, sf = G.quantize_rows(d, 1.0)
    st = rule2(codes, sf, d, 1.0, "row", "exact", bound)
    assert st["scale_acc_allowance"] == 0 and st["scale_boundary_mismatch"] == 0
