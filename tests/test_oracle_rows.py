"""Pins for the oracle's row targets (vllm-metal release v0.4.0, Summary).

The sampled row of prefill segment j is cu_seqlens[num_decode + j + 1] - 1;
decode rows are the leading one-token segments; an explicit logits_indices
list replaces the sampled rows; logits_cu_seqlens describes the compacted
logits layout.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import ref_numpy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rows.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"][:20])
def test_rows_golden(case):
    st, idx, lcu = oracle.rows(case["cu_seqlens"], case["num_decode"], case["num_tokens"],
                               case.get("logits_indices"))
    assert st == oracle.OK
    assert idx.tolist() == case["gather_indices"]
    assert lcu.tolist() == case["logits_cu_seqlens"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"][:20])
def test_rows_shift_by_one_fails(case):
    """Off-by-one control (mlxcel PR #1969: shifting the slice by one row
    must fail): the golden values reject a shifted row list."""
    _, idx, _ = oracle.rows(case["cu_seqlens"], case["num_decode"], case["num_tokens"],
                            case.get("logits_indices"))
    for shift in (-1, 1):
        assert (idx + shift).tolist() != case["gather_indices"]


def test_qwen_shape_closed_form():
    """40 prefills of 2048 tokens: the last rows are 2047 + 2048 j."""
    cu = np.arange(41, dtype=np.int32) * 2048
    st, idx, lcu = oracle.rows(cu, 0, 40 * 2048)
    assert st == oracle.OK
    assert np.array_equal(idx, 2047 + 2048 * np.arange(40))
    assert np.array_equal(lcu, np.arange(41))


def test_pure_decode_is_identity():
    """Pure-decode steps select every row in order (vllm-metal release:
    pure decode is unchanged)."""
    S = 17
    cu = np.arange(S + 1, dtype=np.int32)
    st, idx, lcu = oracle.rows(cu, S, S)
    assert st == oracle.OK
    assert np.array_equal(idx, np.arange(S))
    assert np.array_equal(lcu, np.arange(S + 1))


@pytest.mark.parametrize("cu,nd,T,ex,want", [
    ([0, 2, 1], 0, 5, None, oracle.ERR_LAYOUT),          # decreasing
    ([1, 2, 3], 0, 5, None, oracle.ERR_LAYOUT),          # cu[0] != 0
    ([0, 2, 3], 1, 5, None, oracle.ERR_LAYOUT),          # decode segment of 2 tokens
    ([0, 1, 1, 4], 1, 5, None, oracle.ERR_LAYOUT),       # empty segment (sampled mode)
    ([0, 1, 1, 4], 1, 5, [0, 3], oracle.OK),             # empty segment is fine explicitly
    ([0, 3, 6], 0, 5, None, oracle.ERR_LAYOUT),          # cu[S] beyond num_tokens
    ([0, 3, 5], 0, 5, [0, 5], oracle.ERR_INDEX),         # explicit index out of range
    ([0, 3, 5], 0, 5, [-1], oracle.ERR_INDEX),
    ([0, 1, 2], 3, 5, None, oracle.ERR_LAYOUT),          # num_decode > S
])
def test_rows_errors(cu, nd, T, ex, want):
    st, _, _ = oracle.rows(cu, nd, T, ex)
    assert st == want


def test_rows_random_vs_numpy():
    g = np.random.default_rng(7)
    for _ in range(200):
        nd = int(g.integers(0, 6))
        lens = [1] * nd + list(g.integers(1, 50, size=int(g.integers(0, 8))))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        T = int(cu[-1]) + int(g.integers(0, 3))
        if T == 0:
            continue
        st, idx, lcu = oracle.rows(cu, nd, T)
        assert st == oracle.OK
        i2, l2 = ref_numpy.rows(cu)
        assert np.array_equal(idx, i2) and np.array_equal(lcu, l2)
        ex = np.sort(g.choice(T, size=int(g.integers(1, T + 1)), replace=False)).astype(np.int32)
        st, idx, lcu = oracle.rows(cu, nd, T, ex)
        assert st == oracle.OK
        i2, l2 = ref_numpy.rows(cu, ex)
        assert np.array_equal(idx, i2) and np.array_equal(lcu, l2)
