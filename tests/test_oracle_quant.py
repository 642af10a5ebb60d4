"""Pins for the oracle's dequantisation of affine group-quantised head
weights (the 4-bit models measured in mlxcel PR #1969, description).

Format read for them: W[v][k] = scale[v][k // group] * q(v, k) +
bias[v][k // group], with q an unsigned `bits`-bit integer packed
little-endian into 32-bit words, scale and bias bf16."""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant.json")
BF16_ONE = 0x3F80


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _pack_by_hand(qint: np.ndarray, bits: int) -> np.ndarray:
    """Pack one integer at a time with Python ints: element k goes to bit
    position k * bits of the row, counted from bit 0 of word 0."""
    V, H = qint.shape
    words = (H * bits + 31) // 32
    out = np.zeros((V, words), dtype=np.uint32)
    for v in range(V):
        acc = 0
        for k in range(H):
            acc |= int(qint[v, k]) << (k * bits)
        for w in range(words):
            out[v, w] = (acc >> (32 * w)) & 0xFFFFFFFF
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_worked_cases(case):
    W = oracle.dequant(np.array(case["q"], dtype=np.uint32), np.array(case["scales"], dtype=np.uint16),
                       np.array(case["biases"], dtype=np.uint16), case["bits"], case["group"], case["hidden"])
    assert np.array_equal(W, np.array(case["weights"], dtype=np.float64))


@pytest.mark.parametrize("bits", [4, 8])
def test_unit_scale_zero_bias_returns_the_integers(bits):
    """scale 1, bias 0: the weights are the packed integers themselves; a
    wrong word, bit offset or mask fails."""
    g = synth.rng(11 + bits)
    V, H, G = 5, 192, 64
    qint = g.integers(0, 1 << bits, size=(V, H))
    q = _pack_by_hand(qint, bits)
    s = np.full((V, H // G), BF16_ONE, dtype=np.uint16)
    b = np.zeros((V, H // G), dtype=np.uint16)
    assert np.array_equal(oracle.dequant(q, s, b, bits, G, H), qint.astype(np.float64))


@pytest.mark.parametrize("group", [32, 64, 128])
def test_one_group_scaled_at_a_time(group):
    """All q = 1, bias 0, and a scale that is 1 in group j only: exactly the
    columns [j*group, (j+1)*group) of that row are 1, all others 0."""
    V, H, bits = 3, 512, 4
    q = _pack_by_hand(np.ones((V, H), dtype=np.int64), bits)
    b = np.zeros((V, H // group), dtype=np.uint16)
    for j in range(H // group):
        s = np.zeros((V, H // group), dtype=np.uint16)
        s[1, j] = BF16_ONE
        W = oracle.dequant(q, s, b, bits, group, H)
        want = np.zeros((V, H))
        want[1, j * group:(j + 1) * group] = 1.0
        assert np.array_equal(W, want)


def test_zero_codes_give_the_bias():
    """q = 0 everywhere: every weight equals its group's bias, whatever the
    scale."""
    g = synth.rng(17)
    V, H, G = 4, 256, 64
    q = np.zeros((V, H * 4 // 32), dtype=np.uint32)
    s = synth.normal_bf16(g, (V, H // G))
    b = synth.normal_bf16(g, (V, H // G))
    W = oracle.dequant(q, s, b, 4, G, H)
    assert np.array_equal(W, np.repeat(synth.bf16_bits_to_f32(b).astype(np.float64), G, axis=1))


def test_padded_rows():
    """Row pitches wider than the data (extra words and groups) are skipped."""
    g = synth.rng(19)
    V, H, G = 3, 128, 64
    qint = g.integers(0, 16, size=(V, H))
    q = _pack_by_hand(qint, 4)
    qpad = np.concatenate([q, np.full((V, 3), 0xFFFFFFFF, dtype=np.uint32)], axis=1)
    s = np.full((V, 4), BF16_ONE, dtype=np.uint16)
    b = np.zeros((V, 4), dtype=np.uint16)
    assert np.array_equal(oracle.dequant(qpad, s, b, 4, G, H), qint.astype(np.float64))


def test_signed_integer_head_is_exact():
    """scale 1, bias -8 maps 4-bit codes to the signed integers -8..7; with
    small integer hidden states the quantised head equals integer matmul
    exactly."""
    g = synth.rng(23)
    T, V, H, G = 9, 70, 128, 64
    qint = g.integers(0, 16, size=(V, H))
    q = _pack_by_hand(qint, 4)
    s = np.full((V, H // G), BF16_ONE, dtype=np.uint16)
    b = np.full((V, H // G), synth.f32_to_bf16_bits(np.float32(-8.0)), dtype=np.uint16)
    hid = synth.small_int_bf16(29, (T, H))
    idx = np.array([8, 0, 4, 4], dtype=np.int32)
    Z = oracle.head(hid, oracle.dequant(q, s, b, 4, G, H), idx)
    want = synth.bf16_bits_to_f32(hid).astype(np.int64)[idx] @ (qint - 8).T
    assert np.array_equal(Z, want.astype(np.float64))
