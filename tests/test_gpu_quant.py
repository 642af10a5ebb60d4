"""GPU parity of the quantised-weight head (lmhead_gather_project_q,
lmhead_logprobs_q) with the f64 oracle on exactly dequantised weights
(mlxcel PR #1969, description: the measured models are 4-bit; vllm-metal
release v0.4.0, Summary, for the row selection).

Bar. The library rounds every dequantised weight once to bf16 before its
bf16 MFMA with fp32 accumulation, so against the exact f64 head each logit
may differ by the weight rounding, at most 2**-8 * sum_k |h_k| |w_k| (bf16
keeps 8 significant bits), plus the accumulation error the dense bf16 head
is held to (2e-3 of the row's max |logit|); that sum is the tolerance here,
with sum_k |h_k| |w_k| computed by the oracle. Tighter, bitwise: the
quantised kernels equal the dense bf16 kernels run on the same weights
dequantised in fp32 and rounded to bf16, with the hidden index permuted into
the quantised kernels' summation order; the two quantised kernels equal each
other; and selective rows equal the same rows of the full projection."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_bits, bf16_tensor, check_reduce, i32_tensor

pytestmark = pytest.mark.gpu

TOL = 2e-3
U_BF16 = 2.0 ** -8


def _qweight(d, dev=None):
    dev = dev or torch.device("cuda:0")
    q = torch.from_numpy(d["q"].view(np.int32)).to(dev)
    return lmh.QuantizedWeight(q, bf16_tensor(d["scales"]), bf16_tensor(d["biases"]), d["bits"],
                               d["group"])


def _exact_weights(d):
    return oracle.dequant(d["q"], d["scales"], d["biases"], d["bits"], d["group"], d["hidden_dim"])


def _rounded_weights_bits(d):
    """The library's stated dequantisation, done on the host: fma(scale, code,
    bias) in fp32 (the product is exact, so a float32 multiply then add is the
    same single rounding), then bf16 nearest even."""
    bits, group, H = d["bits"], d["group"], d["hidden_dim"]
    per = 32 // bits
    words = d["q"][:, :H // per]
    shifts = (np.arange(per, dtype=np.uint32) * np.uint32(bits))[None, None, :]
    codes = ((words[:, :, None] >> shifts) & np.uint32((1 << bits) - 1)).reshape(words.shape[0], H)
    s = np.repeat(synth.bf16_bits_to_f32(d["scales"][:, :H // group]), group, axis=1)
    b = np.repeat(synth.bf16_bits_to_f32(d["biases"][:, :H // group]), group, axis=1)
    w = (s * codes.astype(np.float32)).astype(np.float32) + b
    return synth.f32_to_bf16_bits(w.astype(np.float32))


def _quant_order(H, bits):
    """perm[p] = the hidden index that the quantised kernels place at position
    p of the dense kernels' order (MFMA k-step p // 32, lane quarter
    (p // 8) % 4, element p % 8): runs of QB = 512 / bits elements, k-step s
    of a run taking elements QB/4 * quarter + 8 * s .. + 7."""
    qb = 512 // bits
    spb = qb // 32
    p = np.arange(H)
    t, quarter, e = p // 32, (p // 8) % 4, p % 8
    return (t // spb) * qb + quarter * (qb // 4) + (t % spb) * 8 + e


def _tol(hid_f64_rows, W_exact, z_ref):
    A = oracle.head(np.abs(hid_f64_rows), np.abs(W_exact), np.arange(hid_f64_rows.shape[0], dtype=np.int32))
    return U_BF16 * (1 + 2.0 ** -15) * A + TOL * np.abs(z_ref).max(axis=1, keepdims=True)


def _check_vs_oracle(z, hid_bits, idx, W_exact):
    rows = synth.bf16_bits_to_f32(hid_bits).astype(np.float64)[idx]
    z_ref = oracle.head(rows, W_exact, np.arange(len(idx), dtype=np.int32))
    err = np.abs(z.astype(np.float64) - z_ref)
    tol = _tol(rows, W_exact, z_ref)
    assert np.all(err <= tol), float((err / tol).max())
    return z_ref


CASES = [  # (bits, group, H, V)
    (4, 64, 256, 1000), (4, 32, 384, 1001), (4, 128, 128, 4096), (4, 64, 1024, 2053),
    (4, 32, 512, 999), (4, 128, 768, 1500),
    (8, 64, 256, 1000), (8, 32, 128, 777), (8, 128, 640, 3000), (8, 32, 512, 2001),
    (8, 128, 1024, 1024),
    # more than 86 groups per row: the tiled kernel loads scales per stage
    (4, 32, 3072, 700), (8, 32, 2816, 500),
    # 4-bit on either side of the 64-wide-stage kernel's 29-group table limit
    # (28 groups there, 32 and 48 on the 32-wide-stage kernel's LDS table)
    (4, 32, 896, 1003), (4, 32, 1024, 1003), (4, 32, 1536, 515),
]


@pytest.mark.parametrize("s_pad", [2, 3])
@pytest.mark.parametrize("variant", [lmh.LMH_HEAD_STREAM, lmh.LMH_HEAD_TILED])
@pytest.mark.parametrize("bits,group,H,V", CASES)
def test_quant_head_vs_oracle(bits, group, H, V, variant, s_pad):
    """Sampled mode over decode and prefill segments, ragged vocab tails,
    hidden sizes with a partial last chunk (384, 640), both kernels; an even
    and an odd scale row pitch (the streaming kernel reads a chunk's scales
    with one vector load when the pitch is even and the hidden size a
    multiple of 256, one value at a time otherwise)."""
    g = synth.rng(bits * 1000 + group + H + V)
    cu = synth.packed_cu_seqlens(5, [3, 40, 1, 17, 9])
    T = int(cu[-1])
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(bits * 7 + H, V, H, bits, group, q_pad_words=4, s_pad=s_pad)
    p = lmh.lmhead_gather_project_q(bf16_tensor(hid), _qweight(d), i32_tensor(cu), 5, variant=variant)
    st, idx, lcu = oracle.rows(cu, 5, T)
    torch.cuda.synchronize()
    assert st == oracle.OK and int(p.device_error.item()) == 0
    assert np.array_equal(p.gather_indices.cpu().numpy(), idx)
    assert np.array_equal(p.logits_cu_seqlens.cpu().numpy(), lcu)
    _check_vs_oracle(p.logits.cpu().numpy(), hid, idx, _exact_weights(d))


@pytest.mark.parametrize("bits,group,H,V", [(4, 64, 256, 1000), (8, 32, 384, 1001), (4, 128, 1024, 4099)])
@pytest.mark.parametrize("R", [1, 16, 64, 65, 300])
def test_quant_equals_dense_on_rounded_weights(bits, group, H, V, R):
    """Bitwise: quantised kernel == dense bf16 kernel on the host-dequantised,
    bf16-rounded weights with the hidden index permuted into the quantised
    summation order (both sides run the same MFMA sequence on the same
    operands)."""
    g = synth.rng(R * 31 + H + bits)
    T = 320
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(R + V, V, H, bits, group)
    ex = g.integers(0, T, size=R).astype(np.int32)
    cu = i32_tensor([0, T])
    zq = lmh.lmhead_gather_project_q(bf16_tensor(hid), _qweight(d), cu, 0,
                                     logits_indices=i32_tensor(ex)).logits
    perm = _quant_order(H, bits)
    wb = _rounded_weights_bits(d)
    hp = np.ascontiguousarray(hid[:, perm])
    wp = np.ascontiguousarray(wb[:, perm])
    zd = lmh.lmhead_gather_project(bf16_tensor(hp), bf16_tensor(wp), cu, 0,
                                   logits_indices=i32_tensor(ex)).logits
    torch.cuda.synchronize()
    assert np.array_equal(zq.cpu().numpy().view(np.uint32), zd.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("bits,group,H", [(4, 64, 512), (8, 128, 512), (4, 32, 512), (4, 32, 1024)])
def test_stream_and_tiled_bitwise_equal(bits, group, H):
    """The streaming and tiled kernels sum in one order: bitwise equal logits
    (4-bit at 16 groups per row takes the 64-wide-stage tiled kernel, at 32
    the 32-wide-stage one)."""
    g = synth.rng(77 + bits + group)
    V, T = 5003, 100
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(78, V, H, bits, group)
    ex = i32_tensor(g.integers(0, T, size=64).astype(np.int32))
    args = (bf16_tensor(hid), _qweight(d), i32_tensor([0, T]), 0)
    a = lmh.lmhead_gather_project_q(*args, logits_indices=ex, variant=lmh.LMH_HEAD_STREAM).logits
    b = lmh.lmhead_gather_project_q(*args, logits_indices=ex, variant=lmh.LMH_HEAD_TILED).logits
    torch.cuda.synchronize()
    assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))


def test_selective_rows_equal_full_rows():
    """mlxcel PR #1969: the head acts per position, so the sampled rows equal
    the same rows of the projection of every position, bit for bit (here the
    sampled rows stream and the full projection is tiled); the row shifted by
    one does not."""
    g = synth.rng(91)
    H, V = 1024, 8192 + 77
    cu = synth.packed_cu_seqlens(4, [200, 33, 500, 2])
    T = int(cu[-1])
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(92, V, H, 4, 64)
    w = _qweight(d)
    sel = lmh.lmhead_gather_project_q(bf16_tensor(hid), w, i32_tensor(cu), 4)
    full = lmh.lmhead_gather_project_q(bf16_tensor(hid), w, i32_tensor(cu), 4,
                                       logits_indices=i32_tensor(np.arange(T, dtype=np.int32)))
    torch.cuda.synchronize()
    st, idx, _ = oracle.rows(cu, 4, T)
    zs = sel.logits.cpu().numpy()
    zf = full.logits.cpu().numpy()
    assert np.array_equal(zs.view(np.uint32), zf[idx].view(np.uint32))
    assert not np.array_equal(zs, zf[np.clip(idx - 1, 0, T - 1)])


def test_bf16_output_and_invalid_rows():
    g = synth.rng(93)
    H, V, T = 256, 3001, 12
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(94, V, H, 8, 64)
    ex = i32_tensor(np.array([0, 12, 5, -1, 11], dtype=np.int32))
    args = (bf16_tensor(hid), _qweight(d), i32_tensor([0, T]), 0)
    f = lmh.lmhead_gather_project_q(*args, logits_indices=ex)
    b = lmh.lmhead_gather_project_q(*args, logits_indices=ex, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    zf = f.logits.cpu().numpy()
    assert np.all(np.isnan(zf[[1, 3]])) and np.all(np.isfinite(zf[[0, 2, 4]]))
    assert int(f.device_error.item()) & lmh.LMH_DEVERR_INDEX
    assert np.array_equal(bf16_bits(b.logits)[[0, 2, 4]], synth.f32_to_bf16_bits(zf[[0, 2, 4]]))


@pytest.mark.parametrize("bits,group", [(4, 64), (4, 128), (8, 64)])
def test_tiled_ragged_invalid_rows(bits, group):
    """300 rows (a partial row tile) of a 5003-token vocabulary (a partial
    vocab tile) through the tiled kernels (4-bit: the 64-wide stages with the
    tile's scale/bias table): rows without a source are NaN and flagged,
    bf16 output is the rounding of fp32, and 40 valid rows equal, bit for
    bit, the same rows from the weight-streaming kernel."""
    g = synth.rng(95 + bits + group)
    H, V, T, R = 1024, 5003, 400, 300
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(96 + group, V, H, bits, group)
    ex = g.integers(0, T, size=R).astype(np.int32)
    bad = np.array([0, 150, 256, 299])
    ex[bad] = [T, -1, T + 3, -2]
    args = (bf16_tensor(hid), _qweight(d), i32_tensor([0, T]), 0)
    f = lmh.lmhead_gather_project_q(*args, logits_indices=i32_tensor(ex), variant=lmh.LMH_HEAD_TILED)
    b = lmh.lmhead_gather_project_q(*args, logits_indices=i32_tensor(ex), variant=lmh.LMH_HEAD_TILED,
                                    out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    zf = f.logits.cpu().numpy()
    good = np.setdiff1d(np.arange(R), bad)
    assert np.all(np.isnan(zf[bad])) and np.all(np.isfinite(zf[good]))
    assert int(f.device_error.item()) & lmh.LMH_DEVERR_INDEX
    assert np.array_equal(bf16_bits(b.logits)[good], synth.f32_to_bf16_bits(zf[good]))
    sel = g.choice(good, size=40, replace=False)
    q = lmh.lmhead_gather_project_q(*args, logits_indices=i32_tensor(ex[sel]), variant=lmh.LMH_HEAD_STREAM)
    torch.cuda.synchronize()
    assert np.array_equal(q.logits.cpu().numpy().view(np.uint32), zf[sel].view(np.uint32))


@pytest.mark.parametrize("bits", [4, 8])
def test_fused_logprobs_q(bits):
    """lmhead_logprobs_q: the reduction of the projected rows matches the
    oracle's reduction of the same logits (exact ids, 1e-5 logprobs), and the
    logits match the oracle head within the quantised bar."""
    g = synth.rng(95 + bits)
    H, V = 1024, synth.VOCAB_QWEN3
    cu = synth.packed_cu_seqlens(8, [64, 300])
    T = int(cu[-1])
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(96, V, H, bits, 64)
    sel = g.integers(0, V, size=len(cu) - 1).astype(np.int32)
    k = 20
    out = lmh.lmhead_logprobs_q(bf16_tensor(hid), _qweight(d), i32_tensor(cu), 8, i32_tensor(sel), k,
                                return_logits=True)
    torch.cuda.synchronize()
    assert int(out.device_error.item()) == 0
    z = np.ascontiguousarray(out.logits.cpu().numpy())
    st, idx, _ = oracle.rows(cu, 8, T)
    lse, slp, ids, lps = oracle.reduce(z, sel, k)
    check_reduce(out, z, sel, k, lse, slp, ids, lps)
    cols = np.sort(synth.rng(97).choice(V, size=3000, replace=False))
    sub = dict(d, q=np.ascontiguousarray(d["q"][cols]), scales=np.ascontiguousarray(d["scales"][cols]),
               biases=np.ascontiguousarray(d["biases"][cols]))
    _check_vs_oracle(np.ascontiguousarray(z[:, cols]), hid, idx, _exact_weights(sub))


@pytest.mark.parametrize("bits", [4, 8])
def test_decode_qwen3_shape_sampled_columns(bits):
    """Decode step at the Qwen3-0.6B head shape (hidden 1024, vocab 151,936,
    32 one-token segments), the launch the benchmark times: sampled columns
    against the oracle."""
    g = synth.rng(98 + bits)
    H, V, R = 1024, synth.VOCAB_QWEN3, 32
    hid = synth.normal_bf16(g, (R, H))
    d = synth.quantized_head(99, V, H, bits, 64)
    cu = synth.packed_cu_seqlens(R, [])
    p = lmh.lmhead_gather_project_q(bf16_tensor(hid), _qweight(d), i32_tensor(cu), R)
    torch.cuda.synchronize()
    z = p.logits.cpu().numpy()
    cols = np.sort(synth.rng(100).choice(V, size=4000, replace=False))
    cols[-1] = V - 1
    sub = dict(d, q=np.ascontiguousarray(d["q"][cols]), scales=np.ascontiguousarray(d["scales"][cols]),
               biases=np.ascontiguousarray(d["biases"][cols]))
    _check_vs_oracle(np.ascontiguousarray(z[:, cols]), hid, np.arange(R, dtype=np.int32), _exact_weights(sub))


@pytest.mark.parametrize("bits", [4, 8])
def test_qwen3_shape_full_rows(bits):
    """The launches the benchmark times at the Qwen3-0.6B head shape (hidden
    1024, vocab 151,936, group 64): the 40 selected rows of 40 prefills of
    2048 (the streaming kernel) and 8 seeded rows of segment 0's 2048-row
    projection (the tiled kernel), every logit of every row against the
    oracle; the selected rows equal, bit for bit, the same rows of the full
    projection."""
    d = synth.selective_head_batch(4100)
    T, H = d["hidden"].shape
    V = synth.VOCAB_QWEN3
    q = synth.quantized_head(4101, V, H, bits, 64)
    hid = bf16_tensor(d["hidden"])
    qw = _qweight(q)
    cu = i32_tensor(d["cu_seqlens"])
    sel = lmh.lmhead_gather_project_q(hid, qw, cu, 0)
    full = lmh.lmhead_gather_project_q(hid, qw, cu, 0, logits_indices=i32_tensor(np.arange(2048))).logits
    torch.cuda.synchronize()
    idx = (2047 + 2048 * np.arange(40)).astype(np.int32)
    w_exact = _exact_weights(q)
    print(f"oracle quantised head ({bits}-bit): 40 x 151936 x 1024", flush=True)
    _check_vs_oracle(sel.logits.cpu().numpy(), d["hidden"], idx, w_exact)
    rows = np.sort(synth.rng(4102).choice(2048, size=8, replace=False)).astype(np.int32)
    rows[-1] = 2047
    print(f"oracle quantised head ({bits}-bit): 8 rows of the 2048-row projection", flush=True)
    zf = full.cpu().numpy()
    _check_vs_oracle(np.ascontiguousarray(zf[rows]), d["hidden"], rows, w_exact)
    assert np.array_equal(zf[2047].view(np.uint32), sel.logits.cpu().numpy()[0].view(np.uint32))
