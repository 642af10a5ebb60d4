"""Pins for the oracle's per-row reduction.

lse = log(sum_v exp(x_v)), logprob(v) = x_v - lse, the selected token's
logprob, and the exact top-K under (value descending, exact ties by
ascending id) -- MTPLX PR #532, Change; openinfer issue #719, Description
and Suggested direction.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth
from oracle import ref_numpy

NINF = -np.inf


def test_constant_row_closed_form():
    for c, V in [(0.0, 1000), (3.5, 248_320), (-7.25, 151_936), (1e3, 17)]:
        x = np.full((1, V), c, dtype=np.float64)
        lse, sel, ids, lp = oracle.reduce(x, np.array([V - 1]), k=4)
        assert abs(lse[0] - (c + math.log(V))) <= 1e-12 * max(1.0, abs(c))
        assert abs(sel[0] + math.log(V)) <= 1e-12 * max(1.0, abs(c))
        assert ids[0].tolist() == [0, 1, 2, 3]           # all tie: ascending ids
        assert np.allclose(lp[0], -math.log(V), atol=1e-12 * max(1.0, abs(c)))


def test_single_finite_entry():
    x = np.full((1, 50), NINF)
    x[0, 31] = -2.5
    lse, sel, ids, lp = oracle.reduce(x, np.array([31]), k=3)
    assert lse[0] == -2.5 and sel[0] == 0.0
    assert ids[0].tolist() == [31, 0, 1]                  # then the -inf ties, ascending
    assert lp[0, 0] == 0.0 and lp[0, 1] == NINF and lp[0, 2] == NINF


def test_two_valued_row_closed_form():
    a, b, n1, n2 = 2.0, -1.0, 3, 997
    x = np.concatenate([np.full(n2, b), np.full(n1, a)])[None, :]
    lse, _, ids, lp = oracle.reduce(x, None, k=4)
    want = math.log(n1 * math.exp(a) + n2 * math.exp(b))
    assert abs(lse[0] - want) <= 1e-13
    assert ids[0].tolist() == [n2, n2 + 1, n2 + 2, 0]
    assert abs(lp[0, 0] - (a - want)) <= 1e-13


def test_all_neg_inf_row():
    x = np.full((1, 10), NINF, dtype=np.float32)
    lse, sel, ids, lp = oracle.reduce(x, np.array([4]), k=3)
    assert lse[0] == NINF
    assert math.isnan(sel[0])
    assert ids[0].tolist() == [0, 1, 2]
    assert np.all(np.isnan(lp[0]))


def test_signed_zero_ties_by_id():
    """-0 == +0 under IEEE equality: they tie and list by ascending id."""
    x = np.array([[-0.0, 0.0, -1.0, -0.0, 0.0]], dtype=np.float32)
    _, _, ids, _ = oracle.reduce(x, None, k=5)
    assert ids[0].tolist() == [0, 1, 3, 4, 2]


def test_selected_out_of_range_is_nan():
    x = np.zeros((3, 8), dtype=np.float32)
    _, sel, _, _ = oracle.reduce(x, np.array([8, -1, 0]), k=0)
    assert math.isnan(sel[0]) and math.isnan(sel[1]) and sel[2] == -math.log(8)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_logprobs_sum_to_one_and_bounds(dt):
    g = synth.rng(11)
    R, V = 6, 1000
    x = synth.normal_f32(g, (R, V), 3.0)
    x = x if dt == "f32" else synth.f32_to_bf16_bits(x)
    lse, _, ids, lp = oracle.reduce(x, None, k=V)
    assert np.all(np.abs(np.exp(lp).sum(axis=1) - 1.0) <= 1e-12)
    xf = ref_numpy.widen(x)
    mx = xf.max(axis=1)
    assert np.all(mx <= lse) and np.all(lse <= mx + math.log(V))
    assert np.all(np.sort(ids, axis=1) == np.arange(V))   # a permutation


@pytest.mark.parametrize("dist", ["normal", "peaked", "gumbel"])
def test_vs_scipy_and_lexsort(dist):
    """Library cross-check: scipy.special.logsumexp and numpy.lexsort."""
    bits, sel = synth.scoring_chunk(77, dist, 20, rows=4, vocab=20_000)
    lse, slp, ids, lp = oracle.reduce(bits, sel, k=20)
    x = ref_numpy.widen(bits)
    assert np.max(np.abs(lse - logsumexp(x, axis=1))) <= 1e-12
    l2, s2, i2, v2 = ref_numpy.reduce(bits, sel, 20)
    assert np.array_equal(ids, i2)
    assert np.max(np.abs(lp - v2)) <= 1e-12
    assert np.max(np.abs(slp - s2)) <= 1e-12


def test_k1_is_first_argmax():
    bits, _ = synth.decode_logits(5, rows=8, vocab=5000)
    x = synth.bf16_bits_to_f32(bits)
    x[3, 10] = x[3, 20] = x[3].max() + 1.0                 # planted tie at the max
    _, _, ids, _ = oracle.reduce(x, None, k=1)
    assert np.array_equal(ids[:, 0], np.argmax(x, axis=1))
    assert ids[3, 0] == 10


def test_topk_logprob_is_value_minus_lse():
    bits, sel = synth.decode_logits(6, rows=4, vocab=3000)
    lse, slp, ids, lp = oracle.reduce(bits, sel, k=5)
    x = ref_numpy.widen(bits)
    for r in range(4):
        assert np.array_equal(lp[r], x[r, ids[r]] - lse[r])
        assert slp[r] == x[r, sel[r]] - lse[r]
