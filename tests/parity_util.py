"""Parity rules between the HIP library's outputs and the oracle (test infrastructure).

Rule 1 (BF16 C / D / dC, amax, dprob): per expert group,
    max |gpu - ref| / max |ref|  <= 1e-2   (ref: the oracle's float64 value).
Rule 2 (E4M3 D / D_col): >= 99.9 % of elements within 1 E4M3 ULP of the
oracle's code; E8M0 scale bytes bit-exact except for blocks whose
norm_const * amax / 448 (float32) lies within 1e-5 relative of a power of two,
where the two sides may round to neighbouring exponents.
"""
from __future__ import annotations

import numpy as np

from oracle import formats as F
from oracle import grouped as G

RULE1_TOL = 1e-2
RULE2_FRAC = 1e-3
BOUNDARY_REL = 1e-5


def rule1(gpu, ref, grp, what=""):
    """Return the worst per-group ratio; raise AssertionError if above tolerance."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    worst = 0.0
    for g in np.unique(grp):
        sel = grp == g
        den = np.abs(ref[sel]).max() if sel.any() else 0.0
        num = np.abs(gpu[sel] - ref[sel]).max() if sel.any() else 0.0
        if den == 0.0:
            assert num == 0.0, f"{what}: group {g} reference is all zero but gpu differs by {num}"
            continue
        worst = max(worst, num / den)
    assert worst <= RULE1_TOL, f"{what}: rule-1 ratio {worst:.3e} > {RULE1_TOL}"
    return worst


def amax_rule(gpu_amax, ref_amax, what="amax"):
    gpu_amax = np.asarray(gpu_amax, np.float64)
    ref_amax = np.asarray(ref_amax, np.float64)
    worst = 0.0
    for g in range(len(ref_amax)):
        if ref_amax[g] == 0:
            assert gpu_amax[g] == 0, f"{what}[{g}]: expected 0, got {gpu_amax[g]}"
        else:
            worst = max(worst, abs(gpu_amax[g] - ref_amax[g]) / ref_amax[g])
    assert worst <= RULE1_TOL, f"{what}: relative error {worst:.3e}"
    return worst


def _ordinal(codes):
    c = np.asarray(codes).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def near_power_of_two(sf32):
    sf = np.asarray(sf32, np.float64)
    out = np.zeros(sf.shape, bool)
    pos = sf > 0
    r = np.round(np.log2(sf[pos]))
    out[pos] = np.abs(sf[pos] / np.exp2(r) - 1.0) < BOUNDARY_REL
    return out


def rule2(gpu_codes, gpu_sf, ref_d64, nc, axis, what=""):
    """Compare E4M3 codes + E8M0 scales for row blocks (axis='row', blocks of 32
    columns) or column blocks (axis='col', blocks of 32 rows; ref rows must be
    whole aligned blocks).  gpu_sf layout: (rows, cols/32) for rows,
    (cols, rows/32) for columns.  Returns a stats dict."""
    if axis == "row":
        ref_codes, ref_sf = G.quantize_rows(ref_d64, nc)
        d32 = ref_d64.astype(np.float32)
        r, n = d32.shape
        amax = np.abs(d32).reshape(r, n // 32, 32).max(axis=2)
        sf_bcast = lambda s: np.repeat(s, 32, axis=1)
    else:
        ref_codes, ref_sf_t = G.quantize_cols(ref_d64, nc)
        ref_sf = ref_sf_t.T                       # (r/32, n)
        gpu_sf = np.asarray(gpu_sf).T
        d32 = ref_d64.astype(np.float32)
        r, n = d32.shape
        amax = np.abs(d32).reshape(r // 32, 32, n).max(axis=1)
        sf_bcast = lambda s: np.repeat(s, 32, axis=0)
    sf32 = (np.float32(nc) * amax.astype(np.float32)) * G.RCP_MAX_E4M3
    gpu_sf = np.asarray(gpu_sf)
    mism = gpu_sf != ref_sf
    allowed = near_power_of_two(sf32) & (np.abs(gpu_sf.astype(int) - ref_sf.astype(int)) == 1)
    bad_sf = mism & ~allowed
    assert not bad_sf.any(), (f"{what}: {int(bad_sf.sum())} scale bytes differ away from a "
                              f"power-of-two boundary, e.g. at {np.argwhere(bad_sf)[:5].tolist()}")
    same = ~sf_bcast(mism)
    ulp = np.abs(_ordinal(gpu_codes) - _ordinal(ref_codes))
    over = (ulp > 1) & same
    # elements of blocks whose scales legitimately differ: compare dequantised values
    if (~same).any():
        gv = F.decode_e4m3(gpu_codes) * F.decode_e8m0(sf_bcast(gpu_sf))
        rv = F.decode_e4m3(ref_codes) * F.decode_e8m0(sf_bcast(ref_sf))
        # one E4M3 ULP is at most 1/8 of the magnitude, or the subnormal step 2^-9
        # times the (coarser) block scale
        smax = F.decode_e8m0(np.maximum(sf_bcast(gpu_sf), sf_bcast(ref_sf)))
        tol = np.maximum(np.abs(gv), np.abs(rv)) * 0.125 + smax * 2.0 ** -9
        over |= (~same) & (np.abs(gv - rv) > tol * 1.0001)
    n_over = int(over.sum())
    frac = n_over / over.size if over.size else 0.0
    assert frac <= RULE2_FRAC, (f"{what}: {n_over}/{over.size} elements beyond 1 E4M3 ULP "
                                f"(e.g. {np.argwhere(over)[:5].tolist()})")
    return dict(elements=int(over.size), beyond_1ulp=n_over, exact=int((ulp == 0).sum()),
                scale_boundary_mismatch=int(mism.sum()))


def decode_bf16(bits):
    return F.decode_bf16(bits)


def pick_row_blocks(case, nblocks=8, seed=0):
    """Whole 32-row blocks spread over the groups: first, last, the largest
    group, a block holding the end of a group's routed rows, and random ones."""
    po = np.asarray(case.arrays["padded_offsets"])
    vm = int(case.problem["valid_m"])
    total = vm // 32
    rng = np.random.default_rng(seed)
    picks = {0, total - 1}
    starts = np.concatenate([[0], po[:-1]])
    big = int(np.argmax(po - starts))
    picks.add(int(starts[big]) // 32)
    for g in range(len(po)):
        c = int(case.counts[g])
        if c % 32 and c > 0:
            picks.add((int(starts[g]) + c) // 32)      # block with routed rows + padding
            break
    while len(picks) < min(nblocks, total):
        picks.add(int(rng.integers(0, total)))
    blocks = np.array(sorted(picks))
    rows = (blocks[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    return rows
