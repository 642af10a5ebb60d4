"""Planted mistakes in the oracle, on the CPU: each mutant of oracle.c
(a dropped term, a wrong sign or index, a transposed operand, a reversed
tie rule) is compiled on its own and must fail at least one pin. This shows
the pins constrain every step of the oracle rather than re-stating it."""
import json
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rows.json")
QUANT = os.path.join(os.path.dirname(__file__), "golden", "quant.json")
BITMASK = os.path.join(os.path.dirname(__file__), "golden", "bitmask.json")


def _rows_golden_ok(lib):
    with open(GOLDEN) as f:
        for c in json.load(f)["cases"]:
            st, idx, lcu = oracle.rows(c["cu_seqlens"], c["num_decode"], c["num_tokens"],
                                       c.get("logits_indices"), lib=lib)
            if st != 0 or idx.tolist() != c["gather_indices"] or lcu.tolist() != c["logits_cu_seqlens"]:
                return False
    return True


def _head_integer_ok(lib):
    hid = synth.small_int_bf16(1, (7, 48))
    w = synth.small_int_bf16(2, (60, 48))
    idx = np.array([6, 0, 3], dtype=np.int32)
    Z = oracle.head(hid, w, idx, lib=lib)
    hi = synth.bf16_bits_to_f32(hid).astype(np.int64)
    wi = synth.bf16_bits_to_f32(w).astype(np.int64)
    return np.array_equal(Z, (hi[idx] @ wi.T).astype(np.float64))


def _head_one_hot_ok(lib):
    T, H, V = 6, 16, 40
    hid = np.zeros((T, H), dtype=np.float32)
    cols = [0, 5, 15, 7, 1, 9]
    for t, j in enumerate(cols):
        hid[t, j] = 1.0
    w = synth.normal_f32(synth.rng(3), (V, H))
    Z = oracle.head(hid, w, np.arange(T, dtype=np.int32), lib=lib)
    return all(np.array_equal(Z[t], w[:, j].astype(np.float64)) for t, j in enumerate(cols))


def _closed_forms_ok(lib):
    c, V = 3.5, 1000
    lse, sel, ids, lp = oracle.reduce(np.full((1, V), c), np.array([2]), k=3, lib=lib)
    if abs(lse[0] - (c + math.log(V))) > 1e-9 or ids[0].tolist() != [0, 1, 2]:
        return False
    if abs(sel[0] + math.log(V)) > 1e-9:
        return False
    a, b, n1, n2 = 2.0, -1.0, 3, 997
    x = np.concatenate([np.full(n2, b), np.full(n1, a)])[None, :]
    lse, _, ids, lp = oracle.reduce(x, None, k=4, lib=lib)
    want = math.log(n1 * math.exp(a) + n2 * math.exp(b))
    return (abs(lse[0] - want) <= 1e-12 and ids[0].tolist() == [n2, n2 + 1, n2 + 2, 0]
            and abs(lp[0, 0] - (a - want)) <= 1e-12)


def _dequant_golden_ok(lib):
    with open(QUANT) as f:
        for c in json.load(f)["cases"]:
            W = oracle.dequant(np.array(c["q"], dtype=np.uint32), np.array(c["scales"], dtype=np.uint16),
                               np.array(c["biases"], dtype=np.uint16), c["bits"], c["group"], c["hidden"],
                               lib=lib)
            if not np.array_equal(W, np.array(c["weights"], dtype=np.float64)):
                return False
    return True


def _scale_ok(lib):
    hid = synth.small_int_bf16(31, (5, 48))
    w = synth.small_int_bf16(32, (30, 48))
    idx = np.array([4, 0, 2], dtype=np.int32)
    exact = (synth.bf16_bits_to_f32(hid).astype(np.int64)[idx]
             @ synth.bf16_bits_to_f32(w).astype(np.int64).T).astype(np.float64)
    if not np.array_equal(oracle.head(hid, w, idx, lib=lib, scale_mode=oracle.SCALE_MUL, scale=0.5),
                          exact / 2.0):
        return False
    wi = synth.bf16_bits_to_f32(synth.small_int_bf16(34, (40, 64)))
    hid2 = synth.small_int_bf16(33, (6, 64))
    z = oracle.head(hid2, (wi * np.float32(49.0)).astype(np.float32), np.arange(6, dtype=np.int32),
                    lib=lib, scale_mode=oracle.SCALE_DIV, scale=49.0)
    ints = synth.bf16_bits_to_f32(hid2).astype(np.int64) @ wi.astype(np.int64).T
    return np.array_equal(z, ints.astype(np.float64))


def _f16_ok(lib):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    got, want = oracle.widen(h, lib=lib), h.astype(np.float64)
    nan = np.isnan(want)
    return np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan], want[~nan])


def _bitmask_golden_ok(lib):
    with open(BITMASK) as f:
        for c in json.load(f)["cases"]:
            x = synth.normal_f32(synth.rng(81), (c["rows"], c["vocab"]))
            st, Z = oracle.apply_bitmask(x, np.array(c["mask"], dtype=np.uint32), c["logits_cu_seqlens"],
                                         lib=lib)
            if st != 0 or [np.flatnonzero(np.isfinite(z)).tolist() for z in Z] != c["kept"]:
                return False
    return True


def _all_pins_ok(lib):
    return (_rows_golden_ok(lib) and _head_integer_ok(lib) and _head_one_hot_ok(lib)
            and _closed_forms_ok(lib) and _dequant_golden_ok(lib) and _scale_ok(lib)
            and _f16_ok(lib) and _bitmask_golden_ok(lib))


MUTANTS = [
    ("sampled row off by one", "if (idx_out) idx_out[s] = cu[s + 1] - 1;", "if (idx_out) idx_out[s] = cu[s + 1];"),
    ("explicit count <= instead of <", "if (explicit_idx[r] < cu[s]) ++c;", "if (explicit_idx[r] <= cu[s]) ++c;"),
    ("head drops the last term", "for (int64_t k = 0; k < H; ++k)\n                acc +=", "for (int64_t k = 0; k < H - 1; ++k)\n                acc +="),
    ("head transposed weight operand", "widen(W, wdt, v * wld + k)", "widen(W, wdt, k * wld + v)"),
    ("exp of the negated difference", "s += exp(widen(logits, dt, base + v) - m);", "s += exp(m - widen(logits, dt, base + v));"),
    ("lse drops the max", "l = m + log(s);", "l = log(s);"),
    ("ties by descending id", "return (a->id < b->id) ? -1 : (a->id > b->id ? 1 : 0);", "return (a->id > b->id) ? -1 : (a->id < b->id ? 1 : 0);"),
    ("logprob sign flipped", "topk_lp[r * K + i] = e[i].x - l;", "topk_lp[r * K + i] = l - e[i].x;"),
    ("dequant ignores the bit offset", "const uint32_t qv = (word >> (bit % 32)) & mask;", "const uint32_t qv = word & mask;"),
    ("dequant nibbles from the top", "const uint32_t qv = (word >> (bit % 32)) & mask;", "const uint32_t qv = (word >> (32 - bits - bit % 32)) & mask;"),
    ("dequant drops the bias", "* (double)qv +\n                             widen(biases, ORC_BF16, v * s_ld + g);", "* (double)qv;"),
    ("dequant scale and bias swapped", "W64[v * H + k] = widen(scales,", "W64[v * H + k] = widen(biases,"),
    ("dequant group twice as wide", "const int64_t g = k / group;", "const int64_t g = k / (2 * group);"),
    ("multiply mode divides", "for (int64_t i = 0; i < n; ++i) Z[i] = Z[i] * value;", "for (int64_t i = 0; i < n; ++i) Z[i] = Z[i] / value;"),
    ("divide mode by the reciprocal", "for (int64_t i = 0; i < n; ++i) Z[i] = Z[i] / value;", "for (int64_t i = 0; i < n; ++i) Z[i] = Z[i] * (1.0 / value);"),
    ("f16 exponent bias off by one", "v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 26);"),
    ("f16 subnormal scale", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("f16 drops the implicit bit", "v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)m, e - 25);"),
    ("selected logprob adds lse", ": widen(logits, dt, base + t) - l;", ": widen(logits, dt, base + t) + l;"),
    ("bitmask bits read from the top", "if (((word >> (v % 32)) & 1u) == 0)", "if (((word >> (31 - v % 32)) & 1u) == 0)"),
    ("bitmask row of the logits row, not the segment", "mask[s * mask_ld + v / 32]", "mask[r * mask_ld + v / 32]"),
    ("bitmask set bit masks", "if (((word >> (v % 32)) & 1u) == 0)", "if (((word >> (v % 32)) & 1u) != 0)"),
    ("bitmask word index off by one", "mask[s * mask_ld + v / 32]", "mask[s * mask_ld + (v + 1) / 32]"),
]


def test_unmutated_oracle_passes_the_pins():
    assert _all_pins_ok(oracle.load())


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mpath), "-o", so, "-lm"],
                   check=True)
    lib = oracle.load(so)
    assert not _all_pins_ok(lib), f"mutant '{name}' survived every pin"
