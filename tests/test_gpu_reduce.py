"""GPU parity of logprob_reduce with the f64 oracle (MTPLX PR #532, Change;
openinfer issue #719, Suggested direction and Acceptance criteria).

Bar: top-K ids bit-exact on fixed logits; lse, selected and top-K logprobs
within 1e-5 absolute of the f64 oracle; a top-K logprob equals
float32(logit) - lse computed once (bitwise)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_tensor, check_reduce, f32_tensor, i32_tensor

pytestmark = pytest.mark.gpu


def _run(logits_np, sel, k):
    t = bf16_tensor(logits_np) if logits_np.dtype == np.uint16 else f32_tensor(logits_np)
    s = None if sel is None else i32_tensor(sel)
    out = lmh.logprob_reduce(t, s, k)
    ref = oracle.reduce(logits_np, sel, k)
    check_reduce(out, logits_np, sel, k, *ref)
    assert int(out.device_error.item()) == 0
    return out


@pytest.mark.parametrize("sel_mode", ["argmax", "uniform"])
@pytest.mark.parametrize("k", [1, 5])
def test_decode_rows(sel_mode, k):
    """32 x 151,936 bf16 rows of 2*N(0,1) with a +12 peak."""
    print(f"decode rows sel={sel_mode} k={k}", flush=True)
    bits, sel = synth.decode_logits(2000 + k * 10 + (sel_mode == "argmax"), sel_mode=sel_mode)
    out = _run(bits, sel, k)
    if sel_mode == "argmax":
        assert np.array_equal(out.topk_ids.cpu().numpy()[:, 0], sel)


@pytest.mark.parametrize("dist", ["normal", "peaked", "gumbel"])
@pytest.mark.parametrize("k", [0, 1, 20, 128])
def test_scoring_chunk(dist, k):
    """256 x 248,320 bf16 chunks with planted K-th ties and -inf entries."""
    seed = 3000 + 100 * ["normal", "peaked", "gumbel"].index(dist) + k
    print(f"scoring chunk dist={dist} k={k} seed={seed}", flush=True)
    bits, sel = synth.scoring_chunk(seed, dist, k)
    _run(bits, sel, k)


def test_edge_rows():
    """All -inf; 100 finite entries at K=128; constant; -0/+0 ties; a row
    whose K-th value ties across many blocks."""
    V = 248_320
    rows = np.full((5, V), 0x3F80, dtype=np.uint16)          # 1.0 everywhere (constant row 2)
    rows[0, :] = 0xFF80                                       # all -inf
    rows[1, :] = 0xFF80
    pos = synth.rng(5).choice(V, size=100, replace=False)
    rows[1, pos] = synth.f32_to_bf16_bits(synth.normal_f32(synth.rng(6), (100,)))
    rows[3, :] = np.where(np.arange(V) % 2 == 0, 0x8000, 0x0000)   # -0/+0 alternate
    rows[3, 77_777] = 0x3F80
    rows[4, :] = 0xBF80                                        # -1 everywhere ...
    rows[4, ::997] = 0x4000                                    # ... 2.0 every 997th (ties across blocks)
    sel = np.array([0, int(pos[0]), 5, 77_777, V - 1], dtype=np.int32)
    out = _run(rows, sel, 128)
    ids = out.topk_ids.cpu().numpy()
    assert ids[0].tolist() == list(range(128))
    assert ids[2].tolist() == list(range(128))
    assert ids[3, 0] == 77_777 and ids[3, 1:].tolist() == list(range(127))


@pytest.mark.parametrize("V", [1, 40, 64, 65, 999, 1000, 4097, 8192])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ragged_vocab(V, dt):
    """Partial last blocks, tiny vocabularies, K beyond the block count."""
    g = synth.rng(V)
    x = synth.normal_f32(g, (7, V), 2.0)
    x[:, g.integers(0, V, size=3)] = x.max()                   # ties at the top
    ld = -(-V // 8) * 8
    full = np.full((7, ld), -np.inf, dtype=np.float32)
    full[:, :V] = x
    data = synth.f32_to_bf16_bits(full) if dt == "bf16" else full
    t = bf16_tensor(data) if dt == "bf16" else f32_tensor(data)
    t = t[:, :V]
    sel = g.integers(0, V, size=7).astype(np.int32)
    nb = -(-V // 64)
    for k in sorted({0, 1, min(V, 5), min(V, nb), min(V, nb + 1), V if V <= 8192 else 128}):
        if min(k, nb) * 64 > 8192:
            continue
        out = lmh.logprob_reduce(t, i32_tensor(sel), k)
        ref = oracle.reduce(np.ascontiguousarray(data[:, :V]), sel, k)
        check_reduce(out, np.ascontiguousarray(data[:, :V]), sel, k, *ref)


def test_full_row_probabilities_sum_to_one():
    V = 1000
    x = synth.normal_f32(synth.rng(8), (4, V), 3.0)
    out = lmh.logprob_reduce(f32_tensor(x), None, V)
    p = np.exp(out.topk_logprobs.cpu().numpy().astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(p - 1.0) <= 1e-4)
    assert np.all(np.sort(out.topk_ids.cpu().numpy(), axis=1) == np.arange(V))


def test_selected_out_of_range_flags():
    x = synth.normal_f32(synth.rng(9), (3, 500))
    out = lmh.logprob_reduce(f32_tensor(x), i32_tensor([500, -1, 3]), 2)
    torch.cuda.synchronize()
    s = out.selected_logprob.cpu().numpy()
    assert np.isnan(s[0]) and np.isnan(s[1]) and np.isfinite(s[2])
    assert int(out.device_error.item()) & lmh.LMH_DEVERR_INDEX


def test_deterministic():
    bits, sel = synth.scoring_chunk(4242, "gumbel", 20, rows=64)
    t, s = bf16_tensor(bits), i32_tensor(sel)
    a = lmh.logprob_reduce(t, s, 20)
    b = lmh.logprob_reduce(t, s, 20)
    torch.cuda.synchronize()
    for x, y in [(a.lse, b.lse), (a.selected_logprob, b.selected_logprob),
                 (a.topk_ids, b.topk_ids), (a.topk_logprobs, b.topk_logprobs)]:
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_strided_rows():
    """A row pitch larger than the vocabulary (a view into a wider buffer)."""
    V, ld = 151_936, 152_064
    g = synth.rng(10)
    wide = synth.f32_to_bf16_bits(synth.normal_f32(g, (9, ld)))
    t = bf16_tensor(wide)[:, :V]
    sel = g.integers(0, V, size=9).astype(np.int32)
    out = lmh.logprob_reduce(t, i32_tensor(sel), 20)
    data = np.ascontiguousarray(wide[:, :V])
    check_reduce(out, data, sel, 20, *oracle.reduce(data, sel, 20))


def test_zero_rows():
    t = torch.empty((0, 1000), dtype=torch.bfloat16, device="cuda")
    out = lmh.logprob_reduce(t, None, 5)
    torch.cuda.synchronize()
    assert out.lse.numel() == 0
