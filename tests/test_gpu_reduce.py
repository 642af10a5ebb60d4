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
from helpers import as_f32, bf16_tensor, check_reduce, f32_tensor, i32_tensor

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


def _edge_block(V):
    """The edge rows of test_edge_rows, for any V >= 2."""
    rows = np.full((5, V), 0x3F80, dtype=np.uint16)
    rows[0, :] = 0xFF80
    rows[1, :] = 0xFF80
    pos = synth.rng(5).choice(V, size=min(100, V), replace=False)
    rows[1, pos] = synth.f32_to_bf16_bits(synth.normal_f32(synth.rng(6), (pos.size,)))
    rows[3, :] = np.where(np.arange(V) % 2 == 0, 0x8000, 0x0000)
    rows[3, V // 3] = 0x3F80
    rows[4, :] = 0xBF80
    rows[4, ::97] = 0x4000
    return rows


@pytest.mark.parametrize("V,dt,k", [(248_320, "bf16", 20), (248_320, "bf16", 128), (248_320, "bf16", 0),
                                    (128_256, "f32", 20), (1000, "bf16", 5), (4097, "f32", 64),
                                    (65, "bf16", 3), (1, "f32", 1), (8192, "bf16", 8192), (40, "bf16", 1)])
def test_row_path_matches_split_path(V, dt, k):
    """256 rows (one workgroup per row on a 256-CU device) against the same
    rows reduced 100 at a time (split path): bitwise equal lse, selected
    logprobs, ids and logprobs; edge rows included; oracle on sampled rows."""
    print(f"row vs split V={V} dt={dt} k={k}", flush=True)
    g = synth.rng(7000 + V % 1000 + k)
    R = 256
    ld = (V + 7) // 8 * 8            # 16-byte row pitch; the logits are a column view
    if dt == "bf16":
        data = synth.f32_to_bf16_bits(synth.normal_f32(g, (R, V)) * np.float32(2.0))
        if V >= 2:
            data[:5] = _edge_block(V)
        full = np.zeros((R, ld), dtype=np.uint16)
        full[:, :V] = data
        t = bf16_tensor(full)[:, :V]
    else:
        data = synth.normal_f32(g, (R, V)) * np.float32(3.0)
        data[0, :] = -np.inf
        full = np.zeros((R, ld), dtype=np.float32)
        full[:, :V] = data
        t = torch.from_numpy(full).cuda()[:, :V]
    ref_rows = data
    sel = g.integers(0, V, size=R).astype(np.int32)
    sel[7] = V          # out of range: NaN and the index flag, on both paths
    if torch.cuda.get_device_properties(0).multi_processor_count <= R:
        assert lmh.reduce_row_path(R, V, k) and not lmh.reduce_row_path(100, V, k)
    a = lmh.logprob_reduce(t, i32_tensor(sel), k)
    parts = [lmh.logprob_reduce(t[i:i + 100], i32_tensor(sel[i:i + 100]), k) for i in range(0, R, 100)]
    torch.cuda.synchronize()
    assert int(a.device_error.item()) == lmh.LMH_DEVERR_INDEX
    cat = lambda f: torch.cat([getattr(p, f) for p in parts])
    assert torch.equal(a.lse.view(torch.int32), cat("lse").view(torch.int32))
    assert torch.equal(a.selected_logprob.view(torch.int32), cat("selected_logprob").view(torch.int32))
    if k > 0:
        assert torch.equal(a.topk_ids, cat("topk_ids"))
        assert torch.equal(a.topk_logprobs.view(torch.int32), cat("topk_logprobs").view(torch.int32))
    pick = np.array([0, 1, 2, 3, 4, 7, 100, 255])
    ref = oracle.reduce(np.ascontiguousarray(ref_rows[pick]), sel[pick], k)
    sub = lmh.Reduction(a.lse[pick], a.selected_logprob[pick], a.topk_ids[pick], a.topk_logprobs[pick],
                        a.device_error)
    check_reduce(sub, np.ascontiguousarray(ref_rows[pick]), sel[pick], k, *ref)


def _prefetch_rows(V, dt, seed):
    """256 rows that steer the one-workgroup-per-row selection of 16-bit
    logits through each of its branches: the row maximum in the partial last
    block (never prefetched: loaded after the threshold); the top values in
    eight consecutive blocks, all held by one selection thread (its extra
    blocks are loaded after the threshold); 300 scattered blocks tied at the
    top, or four runs of 50 consecutive tied blocks (some with two tied
    entries) under five larger blocks: more tied blocks than the path stages
    whole, so only the lowest-indexed ones needed for K are kept, the cut
    falling inside one selection thread's blocks for the runs; plain rows."""
    g = synth.rng(seed)
    x = synth.normal_f32(g, (256, V), 2.0)
    nb = -(-V // 64)
    for r in range(256):
        kind = r % 4
        if kind == 0:
            x[r, V - 1] = 24.0
            x[r, V - 2] = 23.0
        elif kind == 1:
            b0 = 64 * (16 * (r % (nb // 16)))                   # the first block of a selection thread
            x[r, b0:b0 + 8 * 64:64] = np.arange(8, dtype=np.float32) + 16.0
        elif kind == 2 and r % 8 == 2:
            blocks = g.choice(nb - 1, size=300, replace=False)
            x[r, blocks * 64 + 7] = 12.0
        elif kind == 2:
            runs = 50 * g.choice((nb - 1) // 50, size=4, replace=False)
            blocks = (runs[:, None] + np.arange(50)).ravel()
            x[r, blocks * 64 + 7] = 12.0
            x[r, blocks[::3] * 64 + 40] = 12.0
            above = g.choice(nb - 1, size=5, replace=False)
            x[r, above * 64 + 9] = 30.0
    if dt == "bf16":
        return synth.f32_to_bf16_bits(x)
    return x.astype(np.float16)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("k", [1, 20, 128])
def test_prefetched_candidate_paths(dt, k):
    """Oracle parity on every row, and bitwise equality with the split path
    (its selection runs after a separate streaming launch, from block keys
    in the workspace), for rows built to take each branch."""
    V = 248_280                                              # last block holds 24 entries
    print(f"prefetch paths dt={dt} k={k}", flush=True)
    data = _prefetch_rows(V, dt, 7700 + k)
    g = synth.rng(7800 + k)
    sel = g.integers(0, V, size=256).astype(np.int32)
    ld = (V + 7) // 8 * 8
    if dt == "bf16":
        full = np.zeros((256, ld), dtype=np.uint16)
        full[:, :V] = data
        t = bf16_tensor(full)[:, :V]
    else:
        full = np.zeros((256, ld), dtype=np.float16)
        full[:, :V] = data
        t = torch.from_numpy(full).cuda()[:, :V]
    if torch.cuda.get_device_properties(0).multi_processor_count <= 256:
        assert lmh.reduce_row_path(256, V, k)
    a = lmh.logprob_reduce(t, i32_tensor(sel), k)
    check_reduce(a, data, sel, k, *oracle.reduce(data, sel, k))
    parts = [lmh.logprob_reduce(t[i:i + 100], i32_tensor(sel[i:i + 100]), k) for i in range(0, 256, 100)]
    torch.cuda.synchronize()
    cat = lambda f: torch.cat([getattr(p, f) for p in parts])
    assert torch.equal(a.lse.view(torch.int32), cat("lse").view(torch.int32))
    assert torch.equal(a.topk_ids, cat("topk_ids"))
    assert torch.equal(a.topk_logprobs.view(torch.int32), cat("topk_logprobs").view(torch.int32))
    ids = a.topk_ids.cpu().numpy()
    assert np.all(ids[0::4, 0] == V - 1)                     # the partial block's entry leads


def _order_rows(V, seed):
    """Rows whose block maxima are ordered along the row: rising (the top
    blocks are the row's last), falling (its first), a saw-tooth repeated
    every 4096 logits (equal maxima in every streaming item), rows rounded
    to integers (many equal maxima), the top values in the row's first and
    last blocks, and plain normal rows."""
    g = synth.rng(seed)
    x = synth.normal_f32(g, (256, V), 1.0)
    ramp = np.linspace(-20.0, 20.0, V, dtype=np.float32)
    for r in range(256):
        kind = r % 8
        if kind == 0:
            x[r] = ramp + 0.01 * x[r]
        elif kind == 1:
            x[r] = -ramp + 0.01 * x[r]
        elif kind == 2:
            x[r] = np.tile(np.linspace(0.0, 8.0, 4096, dtype=np.float32), V // 4096 + 1)[:V]
        elif kind == 3:
            x[r] = np.round(x[r])                       # few distinct values: equal block maxima
        elif kind == 4:
            x[r, :64] += 30.0
            x[r, -64:] += 30.0
    return synth.f32_to_bf16_bits(x)


@pytest.mark.parametrize("k", [1, 7, 32, 33])
def test_selection_on_ordered_rows(k):
    """The one-workgroup-per-row reduction on rows whose block maxima are
    ordered along the row: oracle parity on every row and bitwise equality
    with the split path."""
    V = 248_320
    print(f"ordered rows k={k}", flush=True)
    data = _order_rows(V, 7900 + k)
    g = synth.rng(7950 + k)
    sel = g.integers(0, V, size=256).astype(np.int32)
    t = bf16_tensor(data)
    if torch.cuda.get_device_properties(0).multi_processor_count <= 256:
        assert lmh.reduce_row_path(256, V, k)
    a = lmh.logprob_reduce(t, i32_tensor(sel), k)
    check_reduce(a, data, sel, k, *oracle.reduce(data, sel, k))
    parts = [lmh.logprob_reduce(t[i:i + 100], i32_tensor(sel[i:i + 100]), k) for i in range(0, 256, 100)]
    torch.cuda.synchronize()
    cat = lambda f: torch.cat([getattr(p, f) for p in parts])
    assert torch.equal(a.lse.view(torch.int32), cat("lse").view(torch.int32))
    assert torch.equal(a.topk_ids, cat("topk_ids"))
    assert torch.equal(a.topk_logprobs.view(torch.int32), cat("topk_logprobs").view(torch.int32))


def _fp32_bin_rows(V, seed):
    """fp32 rows for the threshold search, which first bins the block-max
    keys on their top 16 bits: 200 blocks with distinct maxima inside one
    16-bit bin above the rest (more than the gather holds: the search goes
    on inside the bin); 300 blocks tied exactly at the top (the same, with
    the tie cut by block index); five finite blocks in a row of -inf (the
    K-th key is -inf's, a bin that does not decode to a finite edge); 100
    distinct maxima in one bin (all of that bin's blocks kept, more than K);
    rows near -60 (negative keys); rows of values near 1e-30 with exact zeros of both
    signs; a rising ramp; plain normal rows."""
    g = synth.rng(seed)
    x = synth.normal_f32(g, (256, V), 2.0)
    nb = -(-V // 64)
    step = np.float32(2.0 ** -19)                   # 16-bit bins at 10.0 are 2^-4 wide
    for r in range(256):
        kind = r % 8
        if kind == 1:
            blocks = g.choice(nb - 1, size=200, replace=False)
            x[r, blocks * 64 + 5] = np.float32(10.0) + step * np.arange(200, dtype=np.float32)
        elif kind == 2:
            blocks = g.choice(nb - 1, size=300, replace=False)
            x[r, blocks * 64 + 11] = 12.0
        elif kind == 3:
            keep = g.choice(nb - 1, size=5, replace=False)
            row = np.full(V, -np.inf, dtype=np.float32)
            for b in keep:
                row[b * 64:b * 64 + 64] = x[r, b * 64:b * 64 + 64]
            x[r] = row
        elif kind == 4:
            blocks = g.choice(nb - 1, size=100, replace=False)
            x[r, blocks * 64 + 30] = np.float32(10.0) + step * g.permutation(100).astype(np.float32)
        elif kind == 5:
            x[r] = np.float32(-60.0) + x[r]          # |lse| stays where an fp32 ulp is below 1e-5
        elif kind == 6:
            x[r] = x[r] * np.float32(1e-30)
            x[r, ::97] = 0.0
            x[r, 1::89] = -0.0
        elif kind == 7:
            x[r] = np.linspace(-30.0, 30.0, V, dtype=np.float32) + np.float32(0.001) * x[r]
    return x


@pytest.mark.parametrize("k", [1, 20, 128])
def test_fp32_threshold_bins(k):
    """fp32 logits of the Llama-3-8B prompt chunk shape (256 x 128,256) on
    rows built for each branch of the threshold search: oracle parity on
    every row, and bitwise equality between the one-workgroup-per-row path
    and the split path."""
    V = 128_256
    print(f"fp32 threshold bins k={k}", flush=True)
    data = _fp32_bin_rows(V, 8100 + k)
    g = synth.rng(8150 + k)
    sel = g.integers(0, V, size=256).astype(np.int32)
    t = f32_tensor(data)
    if torch.cuda.get_device_properties(0).multi_processor_count <= 256:
        assert lmh.reduce_row_path(256, V, k)
    a = lmh.logprob_reduce(t, i32_tensor(sel), k)
    check_reduce(a, data, sel, k, *oracle.reduce(data, sel, k))
    parts = [lmh.logprob_reduce(t[i:i + 100], i32_tensor(sel[i:i + 100]), k) for i in range(0, 256, 100)]
    torch.cuda.synchronize()
    cat = lambda f: torch.cat([getattr(p, f) for p in parts])
    assert torch.equal(a.lse.view(torch.int32), cat("lse").view(torch.int32))
    assert torch.equal(a.topk_ids, cat("topk_ids"))
    assert torch.equal(a.topk_logprobs.view(torch.int32), cat("topk_logprobs").view(torch.int32))


@pytest.mark.parametrize("case", ["chunk_bf16", "ragged_bf16", "f16", "f32"])
def test_full_vocabulary_logprobs(case):
    """k = -1: every token's logprob (openinfer issue #719, Acceptance
    criteria). Each is bitwise float32(x) - lse of the same call, within
    1e-5 of the f64 oracle, and equal to the top-K logprobs of a k = 20 call
    at its ids."""
    print(f"full vocabulary {case}", flush=True)
    g = synth.rng(8200 + len(case))
    if case == "chunk_bf16":
        bits, sel = synth.scoring_chunk(8201, "gumbel", 20)
        host, t = bits, bf16_tensor(bits)
    elif case == "ragged_bf16":
        host = synth.f32_to_bf16_bits(synth.normal_f32(g, (7, 1003), 2.0))
        host[3] = 0xFF80                                  # an all -inf row: NaN logprobs
        padded = np.zeros((7, 1008), dtype=np.uint16)     # 16-byte row pitch
        padded[:, :1003] = host
        t = bf16_tensor(padded)[:, :1003]
        sel = g.integers(0, 1003, size=7).astype(np.int32)
    elif case == "f16":
        host = (synth.normal_f32(g, (40, 151_936), 2.0)).astype(np.float16)
        t = torch.from_numpy(host).cuda()
        sel = g.integers(0, 151_936, size=40).astype(np.int32)
    else:
        host = synth.normal_f32(g, (9, 4100), 3.0)
        t = torch.from_numpy(host).cuda()
        sel = g.integers(0, 4100, size=9).astype(np.int32)
    R, V = host.shape
    full = lmh.logprob_reduce(t, i32_tensor(sel), lmh.LMH_K_FULL)
    top = lmh.logprob_reduce(t, i32_tensor(sel), 20)
    torch.cuda.synchronize()
    lp = full.topk_logprobs.cpu().numpy()
    assert lp.shape == (R, V)
    lse = full.lse.cpu().numpy()
    assert np.array_equal(lse.view(np.uint32), top.lse.cpu().numpy().view(np.uint32))
    x = as_f32(host)
    want = (x - lse[:, None].astype(np.float32)).astype(np.float32)
    same = np.isnan(want) == np.isnan(lp)
    assert np.all(same)
    assert np.array_equal(lp.view(np.uint32)[~np.isnan(want)], want.view(np.uint32)[~np.isnan(want)])
    ref = oracle.full_logprobs(host)
    lse_ref = oracle.reduce(host, None, 0)[0]
    fin = np.isfinite(lse_ref)
    assert np.all(np.abs(lse[fin] - lse_ref[fin]) <= np.maximum(1e-5, np.abs(lse_ref[fin]) * 2.0 ** -23))
    finite = np.isfinite(ref)
    err = np.abs(lp[finite].astype(np.float64) - ref[finite])
    assert np.all(err <= np.maximum(1e-5, np.abs(ref[finite]) * 2.0 ** -23)), float(err.max())
    rows = np.arange(R)[:, None]
    ids = top.topk_ids.cpu().numpy()
    tl = top.topk_logprobs.cpu().numpy()
    ok = ~np.isnan(tl)
    assert np.array_equal(lp[rows, ids][ok].view(np.uint32), tl[ok].view(np.uint32))


def _top1_rows(V, seed):
    """Rows for K = 1, whose answer is the first entry equal to the row
    maximum: the maximum planted in several blocks of different selection
    threads, in two blocks of one thread, twice in one block, in block 0, in
    the partial last block only, in both block 0 and the partial last block;
    constant rows; rows of -inf; -0/+0 rows; plain rows."""
    g = synth.rng(seed)
    x = synth.normal_f32(g, (256, V), 2.0)
    nb = -(-V // 64)
    for r in range(256):
        kind = r % 10
        if kind == 0:
            blocks = np.sort(g.choice(nb - 1, size=5, replace=False))
            x[r, blocks * 64 + g.integers(0, 64, size=5)] = 20.0
        elif kind == 1:
            b0 = 16 * int(g.integers(1, (nb - 1) // 16))          # two blocks of one thread
            x[r, b0 * 64 + 40] = 20.0
            x[r, (b0 + 3) * 64 + 2] = 20.0
        elif kind == 2:
            b = int(g.integers(0, nb - 1))
            x[r, b * 64 + 50] = 20.0
            x[r, b * 64 + 9] = 20.0
        elif kind == 3:
            x[r, 5] = 20.0
        elif kind == 4:
            x[r, V - 3] = 20.0
        elif kind == 5:
            x[r, 63] = 20.0
            x[r, V - 1] = 20.0
        elif kind == 6:
            x[r, :] = 1.5
        elif kind == 7:
            x[r, :] = -np.inf
        elif kind == 8:
            x[r] = np.where(np.arange(V) % 3 == 0, -0.0, 0.0)
            x[r, ::7] = -1.0
    return x


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_top1_rows(dt):
    """K = 1 on rows built for the top-entry shortcut (the prefetched block
    of the lowest thread holding the row maximum) and its fallback (the
    maximum in the partial last block): oracle parity on every row, and
    bitwise equality of the one-workgroup-per-row and split paths."""
    V = 248_280                                              # the last block holds 24 entries
    print(f"top-1 rows dt={dt}", flush=True)
    x = _top1_rows(V, 8400 + (dt == "f16"))
    data = synth.f32_to_bf16_bits(x) if dt == "bf16" else x.astype(np.float16)
    g = synth.rng(8410)
    sel = g.integers(0, V, size=256).astype(np.int32)
    ld = (V + 7) // 8 * 8
    full = np.zeros((256, ld), dtype=data.dtype)
    full[:, :V] = data
    t = (bf16_tensor(full) if dt == "bf16" else torch.from_numpy(full).cuda())[:, :V]
    if torch.cuda.get_device_properties(0).multi_processor_count <= 256:
        assert lmh.reduce_row_path(256, V, 1)
    a = lmh.logprob_reduce(t, i32_tensor(sel), 1)
    check_reduce(a, data, sel, 1, *oracle.reduce(data, sel, 1))
    parts = [lmh.logprob_reduce(t[i:i + 100], i32_tensor(sel[i:i + 100]), 1) for i in range(0, 256, 100)]
    torch.cuda.synchronize()
    cat = lambda f: torch.cat([getattr(p, f) for p in parts])
    assert torch.equal(a.lse.view(torch.int32), cat("lse").view(torch.int32))
    assert torch.equal(a.topk_ids, cat("topk_ids"))
    assert torch.equal(a.topk_logprobs.view(torch.int32), cat("topk_logprobs").view(torch.int32))
    ids = a.topk_ids.cpu().numpy()[:, 0]
    assert np.all(ids[3::10] == 5) and np.all(ids[4::10] == V - 3) and np.all(ids[5::10] == 63)
    assert np.all(ids[6::10] == 0) and np.all(ids[7::10] == 0)
