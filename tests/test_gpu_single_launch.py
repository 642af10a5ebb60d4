"""The single-launch reduction for a few rows (each row spread over several
workgroups, the last one to arrive merging the slices; openinfer issue #719,
Description and Suggested direction), forced at every K it supports through
lmh_debug_reduce_single and taken by logprob_reduce_noalloc at K <= 0,
against logprob_reduce on a workspace (the two-launch split path): lse,
selected logprobs, top-K ids and logprobs bitwise equal, on decode rows, the
Llama-3-8B mixed-batch shape, f16, ragged vocabularies, rows built for the
slice selection's branches (both of its threshold searches: K <= 4 and
K > 4), K = 0 and K = -1, and calls of changing shape in a row (the per-row
counters return to zero); the f64 oracle on the decode rows and the edge
rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_tensor, check_reduce, f32_tensor, i32_tensor

pytestmark = pytest.mark.gpu


def _bitwise(a, b, k):
    torch.cuda.synchronize()
    assert torch.equal(a.lse.view(torch.int32), b.lse.view(torch.int32))
    if a.selected_logprob is not None:
        assert torch.equal(a.selected_logprob.view(torch.int32), b.selected_logprob.view(torch.int32))
    if k != 0:
        if k > 0:
            assert torch.equal(a.topk_ids, b.topk_ids)
        assert torch.equal(a.topk_logprobs.view(torch.int32), b.topk_logprobs.view(torch.int32))
    assert int(a.device_error.item()) == int(b.device_error.item())


_COUNTERS = {}


def _counters():
    if "c" not in _COUNTERS:
        _COUNTERS["c"] = torch.zeros(4096, dtype=torch.int32, device="cuda")
    return _COUNTERS["c"]


def _both(t, sel, k):
    s = None if sel is None else i32_tensor(sel)
    a = lmh.reduce_single(t, s, k, _counters())
    b = lmh.logprob_reduce(t, s, k)
    _bitwise(a, b, k)
    if k <= 1:                                         # the no-workspace entry point (single launch at K <= 0)
        _bitwise(lmh.logprob_reduce_noalloc(t, s, k), b, k)
    return a


def _padded(data, dt):
    """A column view of a matrix with a 16-byte row pitch."""
    R, V = data.shape
    ld = (V + 7) // 8 * 8
    if dt == "bf16":
        full = np.zeros((R, ld), dtype=np.uint16)
        full[:, :V] = data
        return bf16_tensor(full)[:, :V]
    full = np.zeros((R, ld), dtype=np.float32)
    full[:, :V] = data
    return torch.from_numpy(full).cuda()[:, :V]


@pytest.mark.parametrize("k", [1, 5, 20, 32])
def test_decode_rows(k):
    """32 x 151,936 bf16 decode rows (2*N(0,1) with a peak), uniform
    selected ids: bitwise the split path, and the oracle."""
    print(f"single launch decode k={k}", flush=True)
    bits, sel = synth.decode_logits(8200 + k, sel_mode="uniform")
    assert not lmh.reduce_row_path(bits.shape[0], bits.shape[1], k)
    a = _both(bf16_tensor(bits), sel, k)
    check_reduce(a, bits, sel, k, *oracle.reduce(bits, sel, k))


def test_llama_mixed_rows_f32():
    """40 x 128,256 fp32 rows at K = 20 (the Llama-3-8B mixed batch's
    sampled rows), one selected id out of range."""
    print("single launch fp32 40 x 128256", flush=True)
    g = synth.rng(8210)
    x = synth.normal_f32(g, (40, 128_256), 3.0)
    sel = g.integers(0, 128_256, size=40).astype(np.int32)
    sel[3] = 128_256
    a = _both(f32_tensor(x), sel, 20)
    assert int(a.device_error.item()) == lmh.LMH_DEVERR_INDEX
    check_reduce(a, x, sel, 20, *oracle.reduce(x, sel, 20))


def test_f16_rows():
    print("single launch f16", flush=True)
    g = synth.rng(8220)
    x = (synth.normal_f32(g, (16, 151_936), 2.0)).astype(np.float16)
    sel = g.integers(0, 151_936, size=16).astype(np.int32)
    _both(torch.from_numpy(x).cuda(), sel, 5)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("V", [1, 40, 64, 65, 999, 4097, 8192, 12_289, 262_144])
def test_ragged_vocab(V, dt):
    """Vocabularies from one logit to 64 full items, with partial blocks,
    partial items and slices of fewer than four items."""
    print(f"single launch ragged V={V} dt={dt}", flush=True)
    g = synth.rng(8230 + V % 997)
    x = synth.normal_f32(g, (7, V), 2.0)
    data = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    t = _padded(data, dt)
    sel = g.integers(0, V, size=7).astype(np.int32)
    for k in sorted({1, min(5, V), min(32, V)}):
        _both(t, sel, k)


def _edge_rows(V):
    """bf16 rows: all -inf; 100 finite entries among -inf; constant; -0/+0
    alternating with one 1.0; 300 blocks tied at the top; the top values in
    the last partial item; the top values in the first block; a K-th tie
    inside one slice (eight equal maxima in consecutive blocks)."""
    g = synth.rng(8240)
    x = synth.normal_f32(g, (8, V), 2.0)
    nb = -(-V // 64)
    x[0, :] = -np.inf
    x[1, :] = -np.inf
    pos = g.choice(V, size=100, replace=False)
    x[1, pos] = synth.normal_f32(g, (100,), 2.0)
    x[2, :] = 1.0
    x[3, :] = np.where(np.arange(V) % 2 == 0, -0.0, 0.0)
    x[3, 77_777] = 1.0
    blocks = g.choice(nb - 1, size=300, replace=False)
    x[4, blocks * 64 + 7] = 12.0
    x[5, V - 30:] = 20.0 + np.arange(30, dtype=np.float32)
    x[6, :64] = 25.0
    b0 = 64 * 500
    x[7, b0:b0 + 8 * 64:64] = 16.0
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("k", [1, 5, 20, 32])
def test_edge_rows(k):
    V = 151_936 - 40                                   # the last item and block are partial
    print(f"single launch edge rows k={k}", flush=True)
    bits = _edge_rows(V)
    g = synth.rng(8250 + k)
    sel = g.integers(0, V, size=8).astype(np.int32)
    t = _padded(bits, "bf16")
    a = _both(t, sel, k)
    check_reduce(a, bits, sel, k, *oracle.reduce(bits, sel, k))


@pytest.mark.parametrize("k", [0, -1])
def test_lse_only_and_full_vocabulary(k):
    print(f"single launch k={k}", flush=True)
    bits, sel = synth.decode_logits(8260 - k)
    _both(bf16_tensor(bits), sel, k)


def test_changing_shapes_in_a_row():
    """Calls of different row counts, slice counts and K back to back on the
    shared scratch: each equals the split path bitwise (a counter left above
    zero by a call would corrupt the next)."""
    print("single launch changing shapes", flush=True)
    g = synth.rng(8270)
    cases = []
    for R, V, k in [(3, 151_936, 5), (100, 50_000, 32), (1, 262_144, 1), (64, 4097, 20), (3, 151_936, 5)]:
        bits = synth.normal_bf16(g, (R, V), 2.0)
        sel = g.integers(0, V, size=R).astype(np.int32)
        t = _padded(bits, "bf16")
        cases.append((t, sel, k, lmh.reduce_single(t, i32_tensor(sel), k, _counters())))
    for t, sel, k, a in cases:
        b = lmh.logprob_reduce(t, i32_tensor(sel), k)
        _bitwise(a, b, k)


def test_rejects_shapes_off_the_path():
    """Rows that fill the compute units, K above 32 and vocabularies above 64
    items take the other paths: the forcing entry point refuses them."""
    dev = "cuda"
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    for R, V, k in [(cu, 4096, 1), (4, 4096, 33), (4, 64 * 4096 + 8, 1)]:
        t = torch.zeros((R, V), dtype=torch.bfloat16, device=dev)
        with pytest.raises(lmh.LmhError) as e:
            lmh.reduce_single(t, None, k, _counters())
        assert e.value.status == 2                       # LMH_ERR_SHAPE


def test_many_calls_back_to_back():
    """Sixty single-launch calls of varying rows, vocabularies and K queued
    back to back with no synchronisation between them, each compared
    bitwise with the two-launch path afterwards: the device-scope stores,
    the per-row counters and their return to zero hold across consecutive
    launches."""
    print("single launch many calls", flush=True)
    g = synth.rng(8300)
    shapes = [(int(g.integers(1, 65)), int(g.choice([4096, 12_289, 50_000, 151_936])), int(g.integers(0, 33)))
              for _ in range(60)]
    data = {V: synth.normal_bf16(g, (64, V), 2.0) for V in {s[1] for s in shapes}}
    tens = {V: _padded(b, "bf16") for V, b in data.items()}
    runs = []
    for R, V, k in shapes:
        k = min(k, V)
        t = tens[V][:R]
        sel = g.integers(0, V, size=R).astype(np.int32)
        runs.append((t, sel, k, lmh.reduce_single(t, i32_tensor(sel), k, _counters())))
    for t, sel, k, a in runs:
        _bitwise(a, lmh.logprob_reduce(t, i32_tensor(sel), k), k)
    assert int(_counters().abs().sum().item()) == 0
