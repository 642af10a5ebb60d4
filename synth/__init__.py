"""Seeded synthetic inputs shaped like the workloads the pages measure.

This module only draws numbers and lays them out. It holds none of the
method's arithmetic (no projection, no logsumexp, no top-K): both the CPU
oracle and the HIP path receive exactly these arrays.

Conventions
-----------
* RNG: ``numpy.random.Generator(PCG64(seed))``.
* Floating draws are float32; bf16 tensors are made by round-to-nearest-even
  on the float32 bit pattern (``f32_to_bf16_bits``) and are carried as raw
  ``uint16`` arrays. -inf survives the rounding unchanged.
* Packed batches are row-major ``[num_tokens, hidden]``; decode rows come
  first as 1-token segments, then the prefill segments (vllm-metal release
  v0.4.0, Summary: the sampled row of prefill segment j is
  ``cu_seqlens[num_decode + j + 1] - 1``).
* Head weights are ``[vocab, hidden]`` row-major (one row per token id).

Stand-ins: the pages measure on a serving dataset and on trained models that
are not available here. Shapes, dtypes and value distributions follow the
pages' synthetic descriptions; no item of any benchmark suite is reproduced.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64  # logits per prefilter block (MTPLX PR #532, Change)

VOCAB_QWEN3 = 151_936      # Qwen3 head width (vllm-metal release, Summary)
VOCAB_SCORING = 248_320    # prompt-scoring chunk width (MTPLX PR #532, Motivation)
VOCAB_LLAMA3 = 128_256     # Llama-3 vocabulary (mlxcel PR #1969: 128k-152k heads)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return raw bits."""
    u = np.array(a, dtype=np.float32, order="C", copy=True).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)      # NaN inputs are not supported
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen raw bf16 bits to float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_f32(g: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def normal_bf16(g: np.random.Generator, shape, std: float = 1.0,
                chunk_rows: int = 8192) -> np.ndarray:
    """bf16 bits of N(0, std^2), drawn in row chunks to bound host memory."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = f32_to_bf16_bits(normal_f32(g, (r1 - r0, flat.shape[1]), std))
    return out


# ---------------------------------------------------------------------------
# Packed batches
# ---------------------------------------------------------------------------

def packed_cu_seqlens(num_decode: int, prefill_lens) -> np.ndarray:
    """cu_seqlens for ``num_decode`` 1-token segments followed by prefills."""
    lens = [1] * num_decode + list(prefill_lens)
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def tiny_batch(seed: int = 1000):
    """Tiny packed batch: 2 decode rows then prefills of 5, 7 and 9 tokens;
    hidden 64, vocab 1000; fp32 hidden N(0,1) and head N(0, 1/64);
    selected ids uniform in [0, 1000); K = 5."""
    g = rng(seed)
    cu = packed_cu_seqlens(2, [5, 7, 9])
    T, H, V = int(cu[-1]), 64, 1000
    hidden = normal_f32(g, (T, H))
    weight = normal_f32(g, (V, H), std=1.0 / 8.0)
    sel = g.integers(0, V, size=len(cu) - 1, dtype=np.int64).astype(np.int32)
    return dict(cu_seqlens=cu, num_decode=2, hidden=hidden, weight=weight,
                selected=sel, k=5, vocab=V, hidden_dim=H)


# ---------------------------------------------------------------------------
# Logits rows for the reduction
# ---------------------------------------------------------------------------

def decode_logits(seed: int, rows: int = 32, vocab: int = VOCAB_QWEN3,
                  sel_mode: str = "uniform"):
    """Decode-logprob rows: bf16 of 2*N(0,1) with +12 added at one uniform
    position per row (the planted peak). ``sel_mode`` = 'argmax' selects the
    first maximal id of each (rounded) row, 'uniform' a uniform id."""
    g = rng(seed)
    x = normal_f32(g, (rows, vocab), std=2.0)
    peak = g.integers(0, vocab, size=rows)
    x[np.arange(rows), peak] += np.float32(12.0)
    bits = f32_to_bf16_bits(x)
    if sel_mode == "argmax":
        sel = np.argmax(bf16_bits_to_f32(bits), axis=1).astype(np.int32)
    elif sel_mode == "uniform":
        sel = g.integers(0, vocab, size=rows).astype(np.int32)
    else:
        raise ValueError(sel_mode)
    return bits, sel


def _scoring_rows_f32(g, dist: str, rows: int, vocab: int) -> np.ndarray:
    if dist == "normal":
        return normal_f32(g, (rows, vocab))
    if dist == "peaked":
        x = normal_f32(g, (rows, vocab))
        x[np.arange(rows), g.integers(0, vocab, size=rows)] += np.float32(15.0)
        return x
    if dist == "gumbel":
        u = g.random(size=(rows, vocab), dtype=np.float64)
        u = np.clip(u, np.finfo(np.float64).tiny, 1.0 - 1e-16)
        return (-np.log(-np.log(u))).astype(np.float32)
    raise ValueError(dist)


def scoring_chunk(seed: int, dist: str, k: int, rows: int = 256,
                  vocab: int = VOCAB_SCORING, neg_inf_frac: float = 1e-3,
                  plant_ties: bool = True, dtype: str = "bf16"):
    """Prompt-scoring chunk of bf16 logits (raw bits; ``dtype='f16'``: an IEEE
    binary16 array instead) plus uniform selected ids.

    Per row: the distribution's draw, rounded to bf16 (or f16, nearest even); about ``neg_inf_frac``
    of the entries (uniform positions, drawn with replacement) and one whole
    64-logit block set to -inf; then, when 0 < ``k`` < vocab, exact ties
    planted at the K-th value v_K (K-th under value-desc/id-asc): v_K is
    copied to three seeded positions that held less than v_K -- one in a
    different block with an id below the K-th id, one in a block whose
    maximum is below v_K (that block's maximum becomes v_K, so equal block
    maxima meet at the selection boundary), and one anywhere.
    """
    if dtype not in ("bf16", "f16"):
        raise ValueError(dtype)
    g = rng(seed)
    nb = (vocab + BLOCK - 1) // BLOCK
    bits = np.empty((rows, vocab), dtype=np.uint16)
    neg_inf_bits = np.uint16(0xFF80 if dtype == "bf16" else 0xFC00)
    step = 32
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = _scoring_rows_f32(g, dist, r1 - r0, vocab)
        bits[r0:r1] = f32_to_bf16_bits(x) if dtype == "bf16" else x.astype(np.float16).view(np.uint16)
    n_inf = int(round(neg_inf_frac * vocab))
    if n_inf:
        pos = g.integers(0, vocab, size=(rows, n_inf))
        bits[np.arange(rows)[:, None], pos] = neg_inf_bits
    blk = g.integers(0, nb, size=rows)
    for r in range(rows):
        b0 = int(blk[r]) * BLOCK
        bits[r, b0:min(vocab, b0 + BLOCK)] = neg_inf_bits
    if plant_ties and 0 < k < vocab:
        for r in range(rows):
            _plant_ties(g, bits[r], k, dtype)
    sel = g.integers(0, vocab, size=rows).astype(np.int32)
    return (bits if dtype == "bf16" else bits.view(np.float16)), sel


def _plant_ties(g, b: np.ndarray, k: int, dtype: str = "bf16") -> None:
    vocab = b.shape[0]
    xf = (bf16_bits_to_f32(b) if dtype == "bf16" else b.view(np.float16)).astype(np.float64)
    v_k = -np.partition(-xf, k - 1)[k - 1]      # K-th largest value
    if not np.isfinite(v_k):
        return
    n_above = int(np.count_nonzero(xf > v_k))
    id_k = int(np.flatnonzero(xf == v_k)[k - 1 - n_above])
    below = np.flatnonzero(xf < v_k)
    if below.size == 0:
        return
    blk_of = below // BLOCK
    # (1) a position in another block with an id below id_K
    c1 = below[(below < id_k) & (blk_of != id_k // BLOCK)]
    # (2) a position in a block whose maximum is below v_K
    nb = (vocab + BLOCK - 1) // BLOCK
    pad = np.full(nb * BLOCK, -np.inf)
    pad[:vocab] = xf
    bmax = pad.reshape(nb, BLOCK).max(axis=1)
    c2 = below[bmax[blk_of] < v_k]
    picks = []
    if c1.size:
        picks.append(int(c1[g.integers(0, c1.size)]))
    if c2.size:
        picks.append(int(c2[g.integers(0, c2.size)]))
    picks.append(int(below[g.integers(0, below.size)]))
    b[picks] = b[id_k]


# ---------------------------------------------------------------------------
# Head workloads
# ---------------------------------------------------------------------------

def selective_head_batch(seed: int, segments: int = 40, seg_len: int = 2048,
                         hidden_dim: int = 1024, vocab: int = VOCAB_QWEN3):
    """Qwen3-0.6B-shaped packed prefill batch: ``segments`` x ``seg_len``
    tokens, bf16 hidden N(0,1) and bf16 head weights N(0, 1/hidden_dim)."""
    g = rng(seed)
    cu = packed_cu_seqlens(0, [seg_len] * segments)
    T = int(cu[-1])
    hidden = normal_bf16(g, (T, hidden_dim))
    weight = normal_bf16(g, (vocab, hidden_dim), std=float(hidden_dim) ** -0.5)
    return dict(cu_seqlens=cu, num_decode=0, hidden=hidden, weight=weight)


def llama3_head_weight(seed: int, hidden_dim: int = 4096,
                       vocab: int = VOCAB_LLAMA3) -> np.ndarray:
    return normal_bf16(rng(seed), (vocab, hidden_dim),
                       std=float(hidden_dim) ** -0.5)


def mixed_batch(seed: int, hidden_dim: int = 4096, vocab: int = VOCAB_LLAMA3,
                num_decode: int = 32, prefill_lens=(512, 2048) * 4, k: int = 20):
    """Llama-3-8B-shaped mixed step: 32 decode rows then 8 prefills of
    alternating 512 / 2048 tokens; bf16 hidden N(0,1); uniform selected ids
    for the 40 sampled rows; K = 20. The head weight comes from
    ``llama3_head_weight``."""
    g = rng(seed)
    cu = packed_cu_seqlens(num_decode, list(prefill_lens))
    T = int(cu[-1])
    hidden = normal_bf16(g, (T, hidden_dim))
    sel = g.integers(0, vocab, size=len(cu) - 1).astype(np.int32)
    return dict(cu_seqlens=cu, num_decode=num_decode, hidden=hidden,
                selected=sel, k=k)


def prompt_batch(seed: int, hidden_dim: int = 4096, vocab: int = VOCAB_LLAMA3,
                 length: int = 1024, k: int = 20):
    """Prompt-logprob mode: one ``length``-token prompt, every position
    scored (explicit indices 0..length-1). Token ids are uniform; the scored
    token of position t is the prompt's next token, and the last position's
    is a fresh uniform draw."""
    g = rng(seed)
    cu = packed_cu_seqlens(0, [length])
    hidden = normal_bf16(g, (length, hidden_dim))
    tokens = g.integers(0, vocab, size=length).astype(np.int32)
    sel = np.empty(length, dtype=np.int32)
    sel[:-1] = tokens[1:]
    sel[-1] = g.integers(0, vocab)
    idx = np.arange(length, dtype=np.int32)
    return dict(cu_seqlens=cu, num_decode=0, hidden=hidden, selected=sel,
                logits_indices=idx, k=k)


def small_int_bf16(seed: int, shape, lo: int = -4, hi: int = 4) -> np.ndarray:
    """bf16 bits of integers uniform in [lo, hi]; every partial sum of
    products stays an exact integer far below 2**24 for modest widths."""
    g = rng(seed)
    v = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v)


def quantized_head(seed: int, vocab: int, hidden_dim: int, bits: int = 4, group: int = 64,
                   q_pad_words: int = 0, s_pad: int = 0, chunk_rows: int = 16384):
    """A head in affine group-quantised form, as 4-bit MLX models ship it
    (mlxcel PR #1969, description): ``bits``-bit codes uniform in
    [0, 2**bits), packed little-endian into uint32 words [vocab, words +
    q_pad_words] (code k of a row at bit k*bits of the row); bf16 scales and
    biases [vocab, groups + s_pad]. Per group, the scale is
    sigma * (0.28 + 0.08 U) * 15 / (2**bits - 1) and the bias is
    -scale * (2**bits - 1) / 2 * (1 + 0.1 N), sigma = hidden_dim**-0.5: the
    code range spans about +-2.4 sigma, like a group of N(0, sigma^2) weights.
    Padding words are 0xFFFFFFFF and padding scales/biases NaN-free garbage
    (bf16 1.0) so that reading them would show."""
    assert bits in (4, 8) and hidden_dim % group == 0 and (hidden_dim * bits) % 32 == 0
    g = rng(seed)
    per = 32 // bits
    words = hidden_dim // per
    groups = hidden_dim // group
    q = np.full((vocab, words + q_pad_words), 0xFFFFFFFF, dtype=np.uint32)
    for r0 in range(0, vocab, chunk_rows):
        r1 = min(vocab, r0 + chunk_rows)
        codes = g.integers(0, 1 << bits, size=(r1 - r0, words, per), dtype=np.uint32)
        shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))[None, None, :]
        q[r0:r1, :words] = np.bitwise_or.reduce(codes << shifts, axis=2)
    sigma = float(hidden_dim) ** -0.5
    levels = float((1 << bits) - 1)
    scale = sigma * (0.28 + 0.08 * g.random((vocab, groups), dtype=np.float32)) * 15.0 / levels
    bias = -scale * levels / 2.0 * (1.0 + 0.1 * g.standard_normal((vocab, groups), dtype=np.float32))
    s = np.full((vocab, groups + s_pad), 0x3F80, dtype=np.uint16)
    b = np.full((vocab, groups + s_pad), 0x3F80, dtype=np.uint16)
    s[:, :groups] = f32_to_bf16_bits(scale.astype(np.float32))
    b[:, :groups] = f32_to_bf16_bits(bias.astype(np.float32))
    return dict(q=q, scales=s, biases=b, bits=bits, group=group, hidden_dim=hidden_dim)
