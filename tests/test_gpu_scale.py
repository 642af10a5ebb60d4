"""GPU parity of head output scaling and of the bit-exact self-check
(vllm-metal release, Summary: Cohere's logit_scale and Granite's
logits_scaling sit outside the projection; selective logits are kept only
where the selected rows equal the model's own output bit for bit; Testing:
a scaled head the selective path misses is rejected).

Bar: scaled logits within 2e-3 of the scaled f64 oracle relative to the
row's max |logit| (scaling preserves the relative bound); bitwise, the
scaled fp32 logits equal one fp32 multiply or IEEE division of the unscaled
GPU logits; the self-check reports zero differences against the library's
own full projection and the exact count and first position of the
differences against a head it does not reproduce."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_bits, bf16_tensor, check_reduce, f32_tensor, i32_tensor

pytestmark = pytest.mark.gpu

TOL = 2e-3
INT64_MAX = np.iinfo(np.int64).max
SCALES = [(lmh.LMH_SCALE_MUL, 0.0625), (lmh.LMH_SCALE_MUL, 0.3), (lmh.LMH_SCALE_DIV, 8.0),
          (lmh.LMH_SCALE_DIV, 6.0)]


def _close(z, z_ref):
    scale = np.abs(z_ref).max(axis=1, keepdims=True)
    err = np.abs(z.astype(np.float64) - z_ref)
    assert np.all(err <= TOL * scale), float((err / scale).max())


def _host_scaled(z32, mode, s):
    z32 = z32.astype(np.float32)
    return z32 * np.float32(s) if mode == lmh.LMH_SCALE_MUL else z32 / np.float32(s)


def _batch(seed, H=256, V=3001):
    g = synth.rng(seed)
    cu = synth.packed_cu_seqlens(3, [9, 30, 2, 70])
    T = int(cu[-1])
    return g, cu, T, synth.normal_bf16(g, (T, H)), synth.normal_bf16(g, (V, H), H ** -0.5)


@pytest.mark.parametrize("variant", [lmh.LMH_HEAD_STREAM, lmh.LMH_HEAD_TILED])
@pytest.mark.parametrize("mode,s", SCALES)
def test_scaled_dense_head(mode, s, variant):
    g, cu, T, hid, w = _batch(int(s * 100) + mode)
    args = (bf16_tensor(hid), None, i32_tensor(cu), 3)
    head = lmh.HeadSpec(bf16_tensor(w), mode, s)
    p = lmh.lmhead_gather_project_ex(args[0], head, args[2], 3, variant=variant)
    u = lmh.lmhead_gather_project_ex(args[0], lmh.HeadSpec(head.weight), args[2], 3, variant=variant)
    b = lmh.lmhead_gather_project_ex(args[0], head, args[2], 3, variant=variant, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    st, idx, _ = oracle.rows(cu, 3, T)
    z = p.logits.cpu().numpy()
    _close(z, oracle.head(hid, w, idx, scale_mode=mode, scale=s))
    want = _host_scaled(u.logits.cpu().numpy(), mode, s)
    assert np.array_equal(z.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(bf16_bits(b.logits), synth.f32_to_bf16_bits(z))


@pytest.mark.parametrize("mode,s", SCALES[1:3])
def test_scaled_fp32_head(mode, s):
    d = synth.tiny_batch(1000)
    head = lmh.HeadSpec(f32_tensor(d["weight"]), mode, s)
    p = lmh.lmhead_gather_project_ex(f32_tensor(d["hidden"]), head, i32_tensor(d["cu_seqlens"]), d["num_decode"])
    u = lmh.lmhead_gather_project_ex(f32_tensor(d["hidden"]), lmh.HeadSpec(head.weight),
                                     i32_tensor(d["cu_seqlens"]), d["num_decode"])
    torch.cuda.synchronize()
    st, idx, _ = oracle.rows(d["cu_seqlens"], d["num_decode"], d["hidden"].shape[0])
    z = p.logits.cpu().numpy()
    _close(z, oracle.head(d["hidden"], d["weight"], idx, scale_mode=mode, scale=s))
    assert np.array_equal(z.view(np.uint32), _host_scaled(u.logits.cpu().numpy(), mode, s).view(np.uint32))


@pytest.mark.parametrize("variant", [lmh.LMH_HEAD_STREAM, lmh.LMH_HEAD_TILED])
def test_scaled_quantised_head(variant):
    g = synth.rng(51)
    H, V, T = 512, 2003, 80
    hid = synth.normal_bf16(g, (T, H))
    d = synth.quantized_head(52, V, H, 4, 64)
    q = lmh.QuantizedWeight(torch.from_numpy(d["q"].view(np.int32)).cuda(), bf16_tensor(d["scales"]),
                            bf16_tensor(d["biases"]), 4, 64)
    ex = i32_tensor(g.integers(0, T, size=40).astype(np.int32))
    cu = i32_tensor([0, T])
    z = lmh.lmhead_gather_project_ex(bf16_tensor(hid), lmh.HeadSpec(q, lmh.LMH_SCALE_DIV, 6.0), cu, 0,
                                     logits_indices=ex, variant=variant).logits
    u = lmh.lmhead_gather_project_q(bf16_tensor(hid), q, cu, 0, logits_indices=ex, variant=variant).logits
    torch.cuda.synchronize()
    want = _host_scaled(u.cpu().numpy(), lmh.LMH_SCALE_DIV, 6.0)
    assert np.array_equal(z.cpu().numpy().view(np.uint32), want.view(np.uint32))


def _full_and_sampled(head, hid, cu, nd, T):
    full = lmh.lmhead_gather_project_ex(bf16_tensor(hid), head, i32_tensor(cu), nd,
                                        logits_indices=i32_tensor(np.arange(T, dtype=np.int32))).logits
    return full


@pytest.mark.parametrize("quant", [False, True])
def test_selfcheck_passes_on_the_full_projection(quant):
    """The selective rows (streamed, 7 rows) equal the full projection of all
    positions (tiled) bit for bit, scaled or not, dense or quantised."""
    g, cu, T, hid, w = _batch(53, H=512)
    if quant:
        d = synth.quantized_head(54, 3001, 512, 8, 64)
        wt = lmh.QuantizedWeight(torch.from_numpy(d["q"].view(np.int32)).cuda(), bf16_tensor(d["scales"]),
                                 bf16_tensor(d["biases"]), 8, 64)
    else:
        wt = bf16_tensor(w)
    for mode, s in [(lmh.LMH_SCALE_NONE, 1.0), (lmh.LMH_SCALE_DIV, 8.0)]:
        head = lmh.HeadSpec(wt, mode, s)
        full = _full_and_sampled(head, hid, cu, 3, T)
        r = lmh.lmhead_selfcheck(bf16_tensor(hid), head, i32_tensor(cu), full, 3)
        torch.cuda.synchronize()
        assert r.result.cpu().numpy().tolist() == [0, INT64_MAX]
        assert int(r.device_error.item()) == 0


def test_selfcheck_rejects_a_head_it_does_not_reproduce():
    """The model's own output is scaled (divided by 8) but the head given to
    the check is not: every selected logit differs, and the first difference
    is reported at row 0, column 0 (vllm-metal release, Testing)."""
    g, cu, T, hid, w = _batch(55)
    scaled = lmh.HeadSpec(bf16_tensor(w), lmh.LMH_SCALE_DIV, 8.0)
    full = _full_and_sampled(scaled, hid, cu, 3, T)
    r = lmh.lmhead_selfcheck(bf16_tensor(hid), lmh.HeadSpec(scaled.weight), i32_tensor(cu), full, 3)
    torch.cuda.synchronize()
    st, idx, _ = oracle.rows(cu, 3, T)
    f = full.cpu().numpy()[idx]
    mine = lmh.lmhead_gather_project(bf16_tensor(hid), scaled.weight, i32_tensor(cu), 3).logits.cpu().numpy()
    diff = f.view(np.uint32) != mine.view(np.uint32)
    flat = np.flatnonzero(diff)
    assert r.result.cpu().numpy().tolist() == [int(diff.sum()), int(flat[0])]
    assert diff.sum() > 0.99 * diff.size


def test_selfcheck_rejects_shifted_rows():
    """Full logits whose row t holds position t-1's projection (the
    off-by-one of mlxcel PR #1969): the check reports differences, and the
    first one lies in the first row whose source differs."""
    g, cu, T, hid, w = _batch(56)
    head = lmh.HeadSpec(bf16_tensor(w))
    full = _full_and_sampled(head, hid, cu, 3, T)
    shifted = torch.roll(full, 1, dims=0).contiguous()
    r = lmh.lmhead_selfcheck(bf16_tensor(hid), head, i32_tensor(cu), shifted, 3)
    torch.cuda.synchronize()
    res = r.result.cpu().numpy()
    assert res[0] > 0 and res[1] < 3001          # row 0 (source 0 vs the last position) differs


def test_fused_logprobs_with_scaled_head():
    """lmhead_logprobs_ex reduces the scaled logits: its debug logits equal
    the scaled projection bit for bit, and its reduction matches the oracle's
    reduction of those logits."""
    g, cu, T, hid, w = _batch(57, V=5000)
    head = lmh.HeadSpec(bf16_tensor(w), lmh.LMH_SCALE_MUL, 0.3)
    sel = g.integers(0, 5000, size=len(cu) - 1).astype(np.int32)
    out = lmh.lmhead_logprobs_ex(bf16_tensor(hid), head, i32_tensor(cu), 3, i32_tensor(sel), 7,
                                 return_logits=True)
    p = lmh.lmhead_gather_project_ex(bf16_tensor(hid), head, i32_tensor(cu), 3)
    torch.cuda.synchronize()
    z = np.ascontiguousarray(out.logits.cpu().numpy())
    assert np.array_equal(z.view(np.uint32), p.logits.cpu().numpy().view(np.uint32))
    lse, slp, ids, lps = oracle.reduce(z, sel, 7)
    check_reduce(out, z, sel, 7, lse, slp, ids, lps)
