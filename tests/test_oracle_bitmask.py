"""Pins for the oracle's token bitmask on the compacted logits layout
(vllm-metal release v0.4.0, Testing: bitmask application under the compacted
layout): hand-worked fixtures, numpy's unpackbits on random masks, the
identity and all-masked closed forms, a single kept token whose logprob is
exactly 0, and malformed segment bounds."""
import json
import math
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bitmask.json")


def _kept_rows(Z):
    return [np.flatnonzero(np.isfinite(z)).tolist() for z in Z]


def test_golden_fixtures():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = synth.normal_f32(synth.rng(81), (c["rows"], c["vocab"]))
        st, Z = oracle.apply_bitmask(x, np.array(c["mask"], dtype=np.uint32), c["logits_cu_seqlens"])
        assert st == 0, c["name"]
        assert _kept_rows(Z) == c["kept"], c["name"]
        keep = np.isfinite(Z)
        assert np.array_equal(Z[keep], x.astype(np.float64)[keep])


def test_matches_unpackbits():
    """Random masks and segment layouts against numpy's little-endian
    unpackbits of the words' bytes."""
    g = synth.rng(82)
    for V in (1, 31, 32, 33, 1000, 4097):
        W = (V + 31) // 32
        lens = g.integers(0, 4, size=6)
        lcu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        R = int(lcu[-1])
        mask = g.integers(0, 2 ** 32, size=(6, W), dtype=np.uint64).astype(np.uint32)
        x = synth.normal_f32(g, (R, V))
        st, Z = oracle.apply_bitmask(x, mask, lcu)
        assert st == 0
        bits = np.unpackbits(mask.view(np.uint8), axis=1, bitorder="little")[:, :V].astype(bool)
        seg = np.repeat(np.arange(6), lens)
        want = np.where(bits[seg], x.astype(np.float64), -np.inf)
        assert np.array_equal(Z, want)


def test_identity_and_all_masked():
    x = synth.normal_f32(synth.rng(83), (3, 100))
    ones = np.full((3, 4), 0xFFFFFFFF, dtype=np.uint32)
    st, Z = oracle.apply_bitmask(x, ones)
    assert st == 0 and np.array_equal(Z, x.astype(np.float64))
    st, Z = oracle.apply_bitmask(x, np.zeros((3, 4), dtype=np.uint32))
    assert st == 0 and np.all(np.isneginf(Z))
    lse, _, _, _ = oracle.reduce(Z, None, 0)
    assert np.all(np.isneginf(lse))


def test_single_kept_token_has_logprob_zero():
    """One kept token: lse equals its logit and its logprob is exactly 0."""
    x = synth.normal_f32(synth.rng(84), (2, 70))
    mask = np.zeros((2, 3), dtype=np.uint32)
    mask[0, 1] = 1 << 5        # token 37
    mask[1, 2] = 1 << 3        # token 67
    st, Z = oracle.apply_bitmask(x, mask)
    assert st == 0
    lse, sel, ids, lp = oracle.reduce(Z, np.array([37, 67], dtype=np.int32), 1)
    assert lse.tolist() == [float(x[0, 37]), float(x[1, 67])]
    assert ids[:, 0].tolist() == [37, 67] and lp[:, 0].tolist() == [0.0, 0.0]
    assert sel.tolist() == [0.0, 0.0]
    masked_sel = oracle.reduce(Z, np.array([36, 0], dtype=np.int32), 0)[1]
    assert masked_sel.tolist() == [-math.inf, -math.inf]          # a masked token: logprob -inf


def test_malformed_segments_are_reported_and_skipped():
    x = synth.normal_f32(synth.rng(85), (4, 40))
    zero = np.zeros((3, 2), dtype=np.uint32)
    for lcu in ([0, 3, 2, 4], [0, 1, 2, 5], [-1, 1, 2, 4]):
        st, Z = oracle.apply_bitmask(x, zero, lcu)
        assert st == oracle.ERR_LAYOUT
    st, Z = oracle.apply_bitmask(x, zero, [0, 3, 2, 4])   # segment 1 (3 -> 2) is skipped
    assert np.all(np.isneginf(Z[:3])) and np.all(np.isneginf(Z[2:]))
    st, Z = oracle.apply_bitmask(x, zero, [0, 1, 2, 5])   # segment 2 runs past the rows
    assert np.all(np.isneginf(Z[:2])) and np.array_equal(Z[2:], x[2:].astype(np.float64))
