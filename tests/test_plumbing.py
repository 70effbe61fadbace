"""Host-side layout plumbing (no GPU): the word-plane scale layout the C ABI
documents for SFA/SFB -- the byte of row r and K-block kb sits at byte offset
4 * ((kb // 4) * rows + r) + kb % 4."""
import numpy as np
import pytest

pl = pytest.importorskip("moe_grouped_block_amd.plumbing")


@pytest.mark.parametrize("shape", [(7, 16), (3, 5, 8), (1, 4)])
def test_scale_planes_offsets(shape):
    rng = np.random.default_rng(1)
    sf = rng.integers(0, 255, shape, dtype=np.uint8)
    planes = pl.scale_planes(sf).reshape(-1)
    rows = int(np.prod(shape[:-1]))
    logical = sf.reshape(rows, shape[-1])
    for r in range(rows):
        for kb in range(shape[-1]):
            assert planes[4 * ((kb // 4) * rows + r) + kb % 4] == logical[r, kb]


def test_scale_planes_rejects_partial_words():
    with pytest.raises(ValueError):
        pl.scale_planes(np.zeros((4, 6), np.uint8))
