"""The block-max prefilter invariant (MTPLX PR #532, Change): with the
vocabulary viewed as 64-logit blocks, the exact top-K lies inside the K
blocks with the largest maxima, provided equal block maxima are ordered by
ascending block index. The oracle's checker is exercised exhaustively on
tiny rows (so the tie rule is proved by enumeration, not sampled) and on
random rows of the real block size."""
import itertools

import numpy as np
import pytest

import oracle
import synth

VALUES = np.array([-np.inf, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)


def _all_rows(n=8):
    idx = np.array(list(itertools.product(range(len(VALUES)), repeat=n)), dtype=np.int8)
    return VALUES[idx]


@pytest.fixture(scope="module")
def rows8():
    return _all_rows(8)


@pytest.mark.parametrize("block", [2, 3, 4])
def test_exhaustive_tiny_rows(rows8, block):
    """Every row of length 8 over {-inf, -0, +0, 1, 2}, every K, blocks of
    2, 3 (partial last block) and 4."""
    for k in range(0, 9):
        fails, cand = oracle.prefilter_check(rows8, k, block=block)
        assert fails == 0, (block, k)
        assert np.all(cand <= min(8, k * block) if k else cand == 0)
        assert np.all(cand >= min(k, 8))


def test_descending_block_ties_break_the_invariant(rows8):
    """The wrong block tie-break loses ids on some rows: the ascending rule
    is required, not incidental."""
    fails, _ = oracle.prefilter_check(rows8, 2, block=2, block_ties_descending=True)
    assert fails > 0


@pytest.mark.parametrize("dist,k", [("normal", 128), ("peaked", 1), ("gumbel", 20),
                                    ("normal", 1), ("gumbel", 128)])
def test_random_rows_block64(dist, k):
    bits, _ = synth.scoring_chunk(500 + k, dist, k, rows=3, vocab=30_000)
    fails, cand = oracle.prefilter_check(bits, k)
    assert fails == 0
    assert np.all(cand >= k) and np.all(cand <= 64 * k)


def test_partial_last_block_and_k_beyond_blocks():
    """V = 1000 gives 16 blocks, the last 40 wide; K >= nb keeps all blocks."""
    x = synth.normal_f32(synth.rng(9), (4, 1000))
    for k in (1, 5, 15, 16, 17, 100, 1000):
        fails, cand = oracle.prefilter_check(x, k)
        assert fails == 0
        if k >= 16:
            # every block is kept; the threshold is the smallest block max
            assert np.all(cand >= k)


def test_page_block_count():
    """248,320 = 3,880 x 64 (MTPLX PR #532, Change)."""
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")) as f:
        items = json.load(f)["items"]
    b = items[0]
    assert -(-b["vocab"] // b["block"]) == b["blocks"] and b["vocab"] % b["block"] == 0
    assert synth.VOCAB_SCORING == b["vocab"] and synth.BLOCK == b["block"]
    assert items[2]["rows"] * items[2]["vocab"] * items[2]["bytes_per"] / 2**20 == items[2]["mib"]
    assert round(items[3]["vocab"] * items[3]["bytes_per"] / 1024) == items[3]["approx_kib"]
    assert round(items[1]["rows"] * items[1]["vocab"] * items[1]["bytes_per"] / 1e6) == 254
