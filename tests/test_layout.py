"""The K-tiled INT8 code layout as the tests restate it (gpu_util): the fast
block-view converters agree with the element formula, the map is a
permutation of the padded buffer, and every 16-row K-tile is one contiguous
1 KiB with the chunk permutation the public header states."""
import numpy as np
import pytest

from gpu_util import padded_rows, tile, tiled_index, untile


@pytest.mark.parametrize("M,K", [(1, 64), (16, 128), (37, 512), (300, 1024)])
def test_block_view_matches_formula(M, K):
    rng = np.random.default_rng(M * K)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    buf = tile(q)
    assert buf.shape == (padded_rows(M), K)
    flat = np.zeros(padded_rows(M) * K, np.int8)
    flat[tiled_index(M, K)] = q
    assert np.array_equal(buf.reshape(-1), flat)
    assert np.array_equal(untile(buf, M, K), q)


def test_index_is_a_permutation_with_contiguous_tiles():
    M, K = 48, 256
    idx = tiled_index(M, K)
    assert np.array_equal(np.sort(idx.reshape(-1)), np.arange(M * K))
    # rows 16..31, K-tile 2: one contiguous KiB at ((1 * 4) + 2) * 1024
    t = idx[16:32, 128:192]
    assert t.min() == 6 * 1024 and t.max() == 7 * 1024 - 1
    # row 16 + 5 (r // 4 == 1): chunk 0 sits in slot 1, chunk 1 in slot 0
    assert idx[21, 128] == 6 * 1024 + 5 * 64 + 16
    assert idx[21, 144] == 6 * 1024 + 5 * 64 + 0
    assert idx[0, 0] == 0 and idx[0, 64] == 1024
