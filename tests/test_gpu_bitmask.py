"""GPU parity of lmhead_apply_bitmask with the oracle (vllm-metal release
v0.4.0, Testing: bitmask application under the compacted layout).

Bar: the masked logits equal the oracle's, element for element (masking is
an exact operation: a kept value is untouched, a masked one is -inf); the
row pitch's padding is never written; malformed segment bounds are skipped
and flagged on both sides; and the whole compacted chain -- gather + head
with several rows per segment, the bitmask through the head's
logits_cu_seqlens, the reduction -- matches the oracle's chain on the same
logits (ids exact, logprobs within 1e-5)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_tensor, check_reduce, i32_tensor

pytestmark = pytest.mark.gpu


def _mask_words(g, S, V):
    """Words drawn among all-clear, all-set and random, so every store path
    of the kernel (vector -inf, nothing, single elements) is taken."""
    W = (V + 31) // 32
    kind = g.integers(0, 3, size=(S, W))
    rnd = g.integers(0, 2 ** 32, size=(S, W), dtype=np.uint64).astype(np.uint32)
    return np.where(kind == 0, np.uint32(0), np.where(kind == 1, np.uint32(0xFFFFFFFF), rnd))


def _logits(g, R, V, dt, pad):
    """Device logits [R][V] in a buffer of row pitch V + pad filled with a
    sentinel, and the host copy of the [R][V] part (oracle input)."""
    x = synth.normal_f32(g, (R, V + pad), 2.0)
    if dt == "bf16":
        host = synth.f32_to_bf16_bits(x)
        full = bf16_tensor(host)
    elif dt == "f16":
        host = x.astype(np.float16)
        full = torch.from_numpy(host).cuda()
    else:
        host = x
        full = torch.from_numpy(host).cuda()
    return full, np.ascontiguousarray(host[:, :V])


def _host(t, dt):
    torch.cuda.synchronize()
    if dt == "bf16":
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.contiguous().cpu().numpy()


@pytest.mark.parametrize("dt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("V", [1, 31, 33, 1000, 151_936])
def test_matches_oracle(dt, V):
    g = synth.rng(9000 + V + len(dt))
    lens = g.integers(0, 3, size=9)
    lcu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    R = int(lcu[-1])
    pad = (-V) % 8 + 8                      # keeps the pitch 16-byte aligned for every dtype
    full, x = _logits(g, R, V, dt, pad)
    mask = _mask_words(g, 9, V)
    before = _host(full, dt).copy()
    err = lmh.lmhead_apply_bitmask(full[:, :V], torch.from_numpy(mask.view(np.int32)).cuda(),
                                   i32_tensor(lcu))
    after = _host(full, dt)
    st, Z = oracle.apply_bitmask(x, mask, lcu)
    assert st == 0 and int(err.item()) == 0
    got = oracle.widen(np.ascontiguousarray(after[:, :V]))
    assert np.array_equal(got, Z)
    assert np.array_equal(after[:, V:], before[:, V:])     # pitch padding untouched


def test_one_row_per_segment_without_cu_seqlens():
    g = synth.rng(9101)
    R, V = 40, 4097
    full, x = _logits(g, R, V, "f32", 7)
    mask = _mask_words(g, R, V)
    lmh.lmhead_apply_bitmask(full[:, :V], torch.from_numpy(mask.view(np.int32)).cuda())
    st, Z = oracle.apply_bitmask(x, mask)
    assert st == 0 and np.array_equal(_host(full, "f32")[:, :V].astype(np.float64), Z)


def test_malformed_segments_skipped_and_flagged():
    g = synth.rng(9102)
    R, V = 4, 300
    for lcu in ([0, 3, 2, 4], [0, 1, 2, 5]):
        full, x = _logits(g, R, V, "bf16", 4)
        mask = np.zeros((3, 10), dtype=np.uint32)
        err = lmh.lmhead_apply_bitmask(full[:, :V], torch.from_numpy(mask.view(np.int32)).cuda(),
                                       i32_tensor(lcu))
        st, Z = oracle.apply_bitmask(x, mask, lcu)
        assert st == oracle.ERR_LAYOUT and int(err.item()) == lmh.LMH_DEVERR_LAYOUT
        assert np.array_equal(oracle.widen(np.ascontiguousarray(_host(full, "bf16")[:, :V])), Z)


def test_compacted_chain_matches_oracle_chain():
    """Explicit logits indices with several rows per segment (prompt-logprob
    style): the head's logits_cu_seqlens route each segment's mask to its
    rows; the reduction of the masked logits matches the oracle's, and a
    segment that keeps one token gets logprob 0 and that token first."""
    g = synth.rng(9103)
    H, V = 256, 5000
    cu = synth.packed_cu_seqlens(2, [9, 14, 6])          # 2 decode rows, 3 prefills
    T = int(cu[-1])
    ex = np.array([0, 1, 2, 5, 10, 11, 12, 20, 24, 30], dtype=np.int32)
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    proj = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 2,
                                     logits_indices=i32_tensor(ex))
    st, idx, lcu = oracle.rows(cu, 2, T, ex)
    assert st == 0 and np.array_equal(proj.logits_cu_seqlens.cpu().numpy(), lcu)
    S = cu.shape[0] - 1
    mask = _mask_words(g, S, V)
    mask[3] = 0
    mask[3, 4097 // 32] = np.uint32(1 << (4097 % 32))   # segment 3 keeps token 4097 only
    z0 = proj.logits.cpu().numpy()                       # the logits the reduction sees, unmasked
    lmh.lmhead_apply_bitmask(proj.logits, torch.from_numpy(mask.view(np.int32)).cuda(),
                             proj.logits_cu_seqlens)
    sel = g.integers(0, V, size=ex.shape[0]).astype(np.int32)
    out = lmh.logprob_reduce(proj.logits, i32_tensor(sel), 20)
    st, Z = oracle.apply_bitmask(z0, mask, lcu)
    assert st == 0
    check_reduce(out, Z.astype(np.float32), sel, 20, *oracle.reduce(Z, sel, 20))
    rows3 = np.arange(lcu[3], lcu[4])
    assert rows3.size > 0
    assert np.all(out.topk_ids.cpu().numpy()[rows3, 0] == 4097)
    assert np.all(out.topk_logprobs.cpu().numpy()[rows3, 0] == 0.0)


@pytest.mark.parametrize("mode", ["explicit", "sampled"])
def test_fused_logprobs_with_mask(mode):
    """lmhead_logprobs_ex with a token bitmask: each chunk's logits are masked
    before they are reduced. The reduced logits (logits_debug) are the
    unmasked logits of the same call without a mask, masked by the oracle
    (exact); the reduction matches the oracle's on them (ids exact, 1e-5).
    Explicit mode: three segments owning 200, 250 and 250 rows, reduced in
    256-row chunks that straddle them; the middle segment's mask clears every
    token (lse -inf, NaN logprobs). Sampled mode: 40 one-row segments, one
    selected token masked."""
    g = synth.rng(9100 + len(mode))
    H, V, K = 256, 3000, 7
    w = bf16_tensor(synth.normal_bf16(g, (V, H), H ** -0.5))
    if mode == "explicit":
        T = 700
        cu = np.array([0, 200, 450, 700], dtype=np.int32)
        ex = np.arange(T, dtype=np.int32)
        S, R = 3, T
    else:
        T = 40 * 37
        cu = (37 * np.arange(41)).astype(np.int32)
        ex = None
        S, R = 40, 40
    hid = bf16_tensor(synth.normal_bf16(g, (T, H)))
    sel = g.integers(0, V, size=R).astype(np.int32)
    mask = _mask_words(g, S, V)
    if mode == "explicit":
        mask[1, :] = 0                                        # a fully masked segment
    else:
        mask[5, sel[5] // 32] &= ~np.uint32(1 << (sel[5] % 32))   # row 5's selected token masked
    head = lmh.HeadSpec(w)
    kw = dict(selected_ids=i32_tensor(sel), k=K, chunk_rows=256, return_logits=True,
              logits_indices=None if ex is None else i32_tensor(ex))
    plain = lmh.lmhead_logprobs_ex(hid, head, i32_tensor(cu), 0, **kw)
    masked = lmh.lmhead_logprobs_ex(hid, head, i32_tensor(cu), 0,
                                    vocab_mask=torch.from_numpy(mask.view(np.int32)).cuda(), **kw)
    torch.cuda.synchronize()
    assert int(masked.device_error.item()) == 0
    lcu = masked.logits_cu_seqlens.cpu().numpy()
    z_plain = np.ascontiguousarray(plain.logits.cpu().numpy())
    z = np.ascontiguousarray(masked.logits.cpu().numpy())
    st, z_ref = oracle.apply_bitmask(z_plain, mask, None if ex is None else lcu)
    assert st == oracle.OK
    assert np.array_equal(np.isneginf(z), np.isneginf(z_ref))
    assert np.array_equal(z.astype(np.float64), z_ref)
    ref = oracle.reduce(z, sel, K)
    check_reduce(masked, z, sel, K, *ref)
    lse = masked.lse.cpu().numpy()
    if mode == "explicit":
        assert np.all(np.isneginf(lse[200:450])) and np.all(np.isfinite(lse[:200]))
        assert np.all(np.isnan(masked.topk_logprobs.cpu().numpy()[200:450]))
    else:
        assert np.isneginf(masked.selected_logprob.cpu().numpy()[5])
