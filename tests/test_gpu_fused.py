"""GPU parity of the fused lmhead_logprobs (vllm-metal release v0.4.0;
mlxcel PR #1969; MTPLX PR #532; openinfer issue #719: prompt logprobs reuse
the device reduction in chunks).

The fused path is checked in two legs: (1) the fp32 logits it reduced
(returned through logits_debug) against the f64 head within 2e-3 of the
row's max |logit|; (2) its reduction against the f64 oracle reduction of
those same fp32 logits -- exact ids, 1e-5 on values. End to end, against the
full f64 chain, logprobs agree within 2 * 2e-3 * max|z| and ids wherever the
K-th to (K+1)-th gap exceeds that tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_tensor, check_reduce, f32_tensor, i32_tensor

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _head_leg(z_gpu, z_ref, tol=TOL):
    scale = np.abs(z_ref).max(axis=1, keepdims=True)
    assert np.all(np.abs(z_gpu.astype(np.float64) - z_ref) <= tol * scale)


def _end_to_end(out, z_ref, sel, k, tol=TOL, rows=None):
    """The fused result against the full f64 chain (the oracle head, then the
    oracle reduction): lse and the selected logprob within 2 * tol * max|z|,
    ids wherever every gap down to the (K+1)-th exceeds that. `rows` picks
    the logits rows z_ref and sel belong to (all rows when None)."""
    lse, slp, ids, lp = oracle.reduce(z_ref, sel, k + 1)
    scale = np.abs(z_ref).max(axis=1)
    e2e = 2 * tol * scale
    pick = slice(None) if rows is None else rows
    assert np.all(np.abs(out.lse.cpu().numpy()[pick] - lse) <= e2e + 1e-5)
    assert np.all(np.abs(out.selected_logprob.cpu().numpy()[pick] - slp) <= e2e + 1e-5)
    gids = out.topk_ids.cpu().numpy()[pick]
    decided = 0
    for r in range(z_ref.shape[0]):
        vals = z_ref[r, ids[r]]
        gaps = vals[:-1] - vals[1:]
        # positions whose order is decided by more than the head tolerance
        if np.all(gaps[:k] > e2e[r]):
            assert np.array_equal(gids[r], ids[r, :k])
            decided += 1
    return decided


def test_tiny_batch_fused():
    d = synth.tiny_batch(1000)
    T = d["hidden"].shape[0]
    out = lmh.lmhead_logprobs(f32_tensor(d["hidden"]), f32_tensor(d["weight"]),
                              i32_tensor(d["cu_seqlens"]), d["num_decode"],
                              i32_tensor(d["selected"]), d["k"], return_logits=True)
    torch.cuda.synchronize()
    st, idx, lcu = oracle.rows(d["cu_seqlens"], d["num_decode"], T)
    assert np.array_equal(out.gather_indices.cpu().numpy(), idx)
    assert np.array_equal(out.logits_cu_seqlens.cpu().numpy(), lcu)
    z = np.ascontiguousarray(out.logits.cpu().numpy())
    z_ref = oracle.head(d["hidden"], d["weight"], idx)
    _head_leg(z, z_ref, 1e-5)
    check_reduce(out, z, d["selected"], d["k"], *oracle.reduce(z, d["selected"], d["k"]))
    _end_to_end(out, z_ref, d["selected"], d["k"], 1e-5)
    # the unfused chain on the same inputs gives the same bits
    p = lmh.lmhead_gather_project(f32_tensor(d["hidden"]), f32_tensor(d["weight"]),
                                  i32_tensor(d["cu_seqlens"]), d["num_decode"])
    r = lmh.logprob_reduce(p.logits, i32_tensor(d["selected"]), d["k"])
    torch.cuda.synchronize()
    assert torch.equal(r.topk_ids, out.topk_ids)
    assert torch.equal(r.lse.view(torch.int32), out.lse.view(torch.int32))


@pytest.fixture(scope="module")
def llama_weight():
    return synth.llama3_head_weight(5000)


def test_mixed_batch_llama_shape(llama_weight):
    """32 decode rows + prefills of 512/2048 (x4), hidden 4096, vocab 128,256,
    K = 20: one 40-row chunk through the weight-streaming head."""
    d = synth.mixed_batch(5001)
    w = llama_weight
    T = d["hidden"].shape[0]
    out = lmh.lmhead_logprobs(bf16_tensor(d["hidden"]), bf16_tensor(w), i32_tensor(d["cu_seqlens"]),
                              d["num_decode"], i32_tensor(d["selected"]), d["k"], return_logits=True)
    torch.cuda.synchronize()
    assert int(out.device_error.item()) == 0
    st, idx, lcu = oracle.rows(d["cu_seqlens"], d["num_decode"], T)
    assert np.array_equal(out.gather_indices.cpu().numpy(), idx)
    assert np.array_equal(out.logits_cu_seqlens.cpu().numpy(), lcu)
    z = np.ascontiguousarray(out.logits.cpu().numpy())
    print("oracle head: 40 x 128256 x 4096", flush=True)
    z_ref = oracle.head(d["hidden"], w, idx)
    _head_leg(z, z_ref)
    check_reduce(out, z, d["selected"], d["k"], *oracle.reduce(z, d["selected"], d["k"]))
    _end_to_end(out, z_ref, d["selected"], d["k"])


def test_prompt_mode_chunks(llama_weight):
    """One 1024-token prompt, every position scored in 256-row chunks."""
    d = synth.prompt_batch(5003)
    w = llama_weight
    hid = bf16_tensor(d["hidden"])
    out = lmh.lmhead_logprobs(hid, bf16_tensor(w), i32_tensor(d["cu_seqlens"]), 0,
                              i32_tensor(d["selected"]), d["k"],
                              logits_indices=i32_tensor(d["logits_indices"]), chunk_rows=256,
                              return_logits=True)
    torch.cuda.synchronize()
    assert int(out.device_error.item()) == 0
    assert out.logits_cu_seqlens.cpu().numpy().tolist() == [0, 1024]
    z = np.ascontiguousarray(out.logits.cpu().numpy())
    check_reduce(out, z, d["selected"], d["k"], *oracle.reduce(z, d["selected"], d["k"]))
    # one row of every 16-row MFMA group (a seeded position inside it), and
    # each chunk's first and last rows, every logit, against the f64 chain
    g = synth.rng(5006)
    rows = np.unique(np.concatenate([16 * np.arange(64) + g.integers(0, 16, size=64),
                                     [0, 255, 256, 511, 512, 767, 768, 1023]]))
    print(f"oracle head: {rows.size} x 128256 x 4096", flush=True)
    z_ref = oracle.head(d["hidden"], w, d["logits_indices"][rows])
    _head_leg(z[rows], z_ref)
    _end_to_end(out, z_ref, d["selected"][rows], d["k"], rows=rows)
    # chunking does not change a row's bits: the same rows projected alone
    alone = lmh.lmhead_gather_project(hid, bf16_tensor(w), i32_tensor(d["cu_seqlens"]), 0,
                                      logits_indices=i32_tensor(rows)).logits
    torch.cuda.synchronize()
    assert np.array_equal(alone.cpu().numpy().view(np.uint32), z[rows].view(np.uint32))


def test_chunk_sizes_agree():
    """Chunks of at most 64 rows reduce with their own streaming pass, larger
    chunks from the tiled head's per-block partials (so with 256-row chunks
    the first 256 rows take the partials and the last 44 their own pass):
    per row, results are bitwise independent of the chunking within each
    kind; across the two, ids are equal and lse agrees to fp32 rounding."""
    g = synth.rng(5004)
    T, H, V = 300, 256, 3000
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = np.arange(T, dtype=np.int32)
    sel = g.integers(0, V, size=T).astype(np.int32)
    outs = {c: lmh.lmhead_logprobs(bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, T]), 0,
                                   i32_tensor(sel), 7, logits_indices=i32_tensor(ex), chunk_rows=c)
            for c in (0, 1, 64, 100, 300)}
    torch.cuda.synchronize()
    lse = {c: o.lse.view(torch.int32).cpu().numpy() for c, o in outs.items()}
    for c in (0, 64, 100, 300):
        assert torch.equal(outs[c].topk_ids, outs[1].topk_ids)
    partials = {0: np.arange(256), 100: np.arange(T), 300: np.arange(T)}
    own_pass = {0: np.arange(256, T), 1: np.arange(T), 64: np.arange(T)}
    for kind in (partials, own_pass):
        rows = set.intersection(*(set(v.tolist()) for v in kind.values()))
        rows = np.array(sorted(rows))
        first = next(iter(kind))
        for c in kind:
            assert np.array_equal(lse[c][rows], lse[first][rows])
    assert float((outs[100].lse - outs[1].lse).abs().max()) <= 1e-5


def test_flagged_rows_fused():
    """A logits row whose source index is out of range is flagged and written
    in full: NaN lse, selected and top-K logprobs, -1 ids; every other row is
    bitwise what it is when that index is valid. Rows 3 and 270 sit in the
    first 256-row chunk (one workgroup per row on a 256-CU device) and in
    the 44-row second chunk (the two-launch path)."""
    g = synth.rng(5005)
    T, H, V, K = 300, 256, 3000, 7
    hid = bf16_tensor(synth.normal_bf16(g, (T, H)))
    w = bf16_tensor(synth.normal_bf16(g, (V, H), H ** -0.5))
    sel = i32_tensor(g.integers(0, V, size=T))
    good = np.arange(T, dtype=np.int32)
    bad = good.copy()
    bad[[3, 270]] = [T + 5, -1]
    runs = [lmh.lmhead_logprobs(hid, w, i32_tensor([0, T]), 0, sel, K, logits_indices=i32_tensor(ex))
            for ex in (good, bad)]
    torch.cuda.synchronize()
    ok, fl = runs
    assert int(ok.device_error.item()) == 0
    assert int(fl.device_error.item()) & lmh.LMH_DEVERR_INDEX
    flagged = np.zeros(T, dtype=bool)
    flagged[[3, 270]] = True
    assert np.all(np.isnan(fl.lse.cpu().numpy()[flagged]))
    assert np.all(np.isnan(fl.selected_logprob.cpu().numpy()[flagged]))
    assert np.all(fl.topk_ids.cpu().numpy()[flagged] == -1)
    assert np.all(np.isnan(fl.topk_logprobs.cpu().numpy()[flagged]))
    assert np.array_equal(fl.gather_indices.cpu().numpy()[flagged], [-1, -1])
    for a, b in ((ok.lse, fl.lse), (ok.selected_logprob, fl.selected_logprob),
                 (ok.topk_logprobs, fl.topk_logprobs)):
        assert np.array_equal(a.cpu().numpy()[~flagged].view(np.uint32), b.cpu().numpy()[~flagged].view(np.uint32))
    assert np.array_equal(ok.topk_ids.cpu().numpy()[~flagged], fl.topk_ids.cpu().numpy()[~flagged])


def test_full_vocabulary_fused():
    """lmhead_logprobs with k = -1 over 300 explicit rows in 256-row chunks:
    every token's logprob of every row, bitwise float32(z) - lse of the fp32
    logits the call reduced, and within 1e-5 of the oracle on those logits."""
    g = synth.rng(5007)
    T, H, V = 300, 256, 3000
    hid = bf16_tensor(synth.normal_bf16(g, (T, H)))
    w = bf16_tensor(synth.normal_bf16(g, (V, H), H ** -0.5))
    sel = g.integers(0, V, size=T).astype(np.int32)
    out = lmh.lmhead_logprobs(hid, w, i32_tensor([0, T]), 0, i32_tensor(sel), lmh.LMH_K_FULL,
                              logits_indices=i32_tensor(np.arange(T)), chunk_rows=256, return_logits=True)
    torch.cuda.synchronize()
    z = np.ascontiguousarray(out.logits.cpu().numpy())
    lp = out.topk_logprobs.cpu().numpy()
    lse = out.lse.cpu().numpy()
    assert lp.shape == (T, V)
    want = (z - lse[:, None]).astype(np.float32)
    assert np.array_equal(lp.view(np.uint32), want.view(np.uint32))
    ref = oracle.full_logprobs(z)
    assert np.max(np.abs(lp - ref)) <= 1e-5


@pytest.mark.parametrize("k,scale", [(20, 0), (0, 0), (5, 2)])
def test_epilogue_partials_match_unfused(llama_weight, k, scale):
    """The Llama-3-8B-shaped prompt (1024 rows in 256-row chunks) with the
    reduction's first pass in the tiled head's epilogue, against the same
    call with that pass run on its own: the reduced logits are bitwise
    equal, ids equal, lse and logprobs within 1e-5; both against the oracle
    on those logits (ids exact, 1e-5). With a divided head the partials are
    those of the scaled logits."""
    d = synth.prompt_batch(5003)
    hid = bf16_tensor(d["hidden"])
    head = lmh.HeadSpec(bf16_tensor(llama_weight), lmh.LMH_SCALE_DIV if scale else lmh.LMH_SCALE_NONE,
                        float(scale) if scale else 1.0)
    kw = dict(selected_ids=i32_tensor(d["selected"]), k=k, logits_indices=i32_tensor(d["logits_indices"]),
              chunk_rows=256, return_logits=True)
    fused = lmh.lmhead_logprobs_ex(hid, head, i32_tensor(d["cu_seqlens"]), 0, epilogue=0, **kw)
    plain = lmh.lmhead_logprobs_ex(hid, head, i32_tensor(d["cu_seqlens"]), 0, epilogue=1, **kw)
    torch.cuda.synchronize()
    assert int(fused.device_error.item()) == 0
    assert torch.equal(fused.logits.view(torch.int32), plain.logits.view(torch.int32))
    assert torch.equal(fused.topk_ids, plain.topk_ids)
    assert float((fused.lse - plain.lse).abs().max()) <= 1e-5
    assert float((fused.selected_logprob - plain.selected_logprob).abs().max()) <= 1e-5
    if k:
        assert float((fused.topk_logprobs - plain.topk_logprobs).abs().max()) <= 1e-5
    z = np.ascontiguousarray(fused.logits.cpu().numpy())
    ref = oracle.reduce(z, d["selected"], k)
    check_reduce(fused, z, d["selected"], k, *ref)


def test_epilogue_partials_full_vocabulary():
    """k = -1 on 300 rows (a 256-row chunk from the epilogue partials, then a
    44-row chunk with its own pass): every logprob bitwise float32(z) - lse
    of the call, lse within 1e-5 of the oracle."""
    g = synth.rng(5008)
    T, H, V = 300, 256, 3000
    hid = bf16_tensor(synth.normal_bf16(g, (T, H)))
    w = bf16_tensor(synth.normal_bf16(g, (V, H), H ** -0.5))
    out = lmh.lmhead_logprobs(hid, w, i32_tensor([0, T]), 0, None, lmh.LMH_K_FULL,
                              logits_indices=i32_tensor(np.arange(T)), chunk_rows=256, return_logits=True)
    torch.cuda.synchronize()
    z = np.ascontiguousarray(out.logits.cpu().numpy())
    lse = out.lse.cpu().numpy()
    assert np.array_equal(out.topk_logprobs.cpu().numpy().view(np.uint32),
                          (z - lse[:, None]).astype(np.float32).view(np.uint32))
    assert np.max(np.abs(lse - oracle.reduce(z, None, 0)[0])) <= 1e-5
