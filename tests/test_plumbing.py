"""Host-side plumbing (no GPU): the generator's scale arrays are already the
C ABI's row-major (rows, K/32) layout, so uploads keep every byte in place,
and a discrete-weight expert's scales are its (N, K/32) slice of SFB."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pl = pytest.importorskip("moe_grouped_block_amd.plumbing")
synth = pytest.importorskip("synth")


def test_scales_upload_row_major():
    case = synth.make_case("fc1_swiglu_l8", seed=3, name="plumb", L=3, K=512, N=128, routing=("topk", 100, 2))
    dev = pl.to_device(case.arrays, device="cpu")
    for k in ("sfa", "sfb"):
        src = case.arrays[k]
        got = dev[k].numpy()
        assert got.shape == src.shape and np.array_equal(got, src)
        # byte kb of row r at r * K/32 + kb
        flat = got.reshape(-1)
        kb = src.shape[-1]
        r, c = 5, 7
        assert flat[r * kb + c] == src.reshape(-1, kb)[r, c]
