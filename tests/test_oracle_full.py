"""Pins for the oracle's full-vocabulary logprobs (openinfer issue #719,
Acceptance criteria: a request of -1 means every token's logprob): each
row's x - lse, in f64.

Closed forms and invariants that a plausible mistake fails: a constant row
gives -ln V everywhere; one finite entry gives 0 there and -inf elsewhere;
exp of every row sums to 1 (a missing or wrong-row lse breaks it); the
values at a row's top-K ids are the top-K logprobs of the reduction; an
all -inf row is NaN."""
import math

import numpy as np

import oracle
import synth

NINF = -np.inf


def test_constant_row():
    for c, V in [(0.0, 1000), (-7.25, 4097)]:
        lp = oracle.full_logprobs(np.full((2, V), c))
        assert np.all(np.abs(lp + math.log(V)) <= 1e-12 * max(1.0, abs(c)))


def test_single_finite_entry():
    x = np.full((1, 70), NINF)
    x[0, 9] = 3.0
    lp = oracle.full_logprobs(x)
    assert lp[0, 9] == 0.0 and np.all(np.isneginf(np.delete(lp[0], 9)))


def test_rows_normalise_and_match_topk():
    g = synth.rng(61)
    x = synth.normal_f32(g, (5, 3000), 3.0)
    x[2] += 40.0                                          # a row far from the others
    lp = oracle.full_logprobs(x)
    assert np.all(np.abs(np.exp(lp).sum(axis=1) - 1.0) <= 1e-12)
    lse, _, ids, tlp = oracle.reduce(x, None, 9)
    rows = np.arange(5)[:, None]
    assert np.array_equal(lp[rows, ids], tlp)
    assert np.array_equal(lp, x.astype(np.float64) - lse[:, None])


def test_bf16_rows_and_all_neg_inf():
    g = synth.rng(62)
    bits = synth.f32_to_bf16_bits(synth.normal_f32(g, (3, 999), 2.0))
    bits[1] = 0xFF80                                       # -inf
    lp = oracle.full_logprobs(bits)
    assert np.all(np.isnan(lp[1]))
    ok = lp[[0, 2]]
    assert np.all(np.abs(np.exp(ok).sum(axis=1) - 1.0) <= 1e-12)
