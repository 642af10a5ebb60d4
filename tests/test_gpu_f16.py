"""GPU parity of logprob_reduce on f16 logits with the f64 oracle (MTPLX PR
#532, Tests: parity on synthetic bf16/f16 logits, exact ties, -inf, K = 0, 1
and 128).

Bar as for bf16: top-K ids bit-exact; lse, selected and top-K logprobs within
1e-5 absolute of the f64 oracle; a top-K logprob equals float32(logit) - lse
rounded once. f16 widens to fp32 exactly, and its 16-bit block keys are a
monotone map of the f16 bits, so equal f16 block maxima tie and ties list by
ascending block index as for bf16."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import check_reduce, i32_tensor

pytestmark = pytest.mark.gpu


def f16_tensor(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16)).to("cuda:0")


def _run(x16, sel, k):
    s = None if sel is None else i32_tensor(sel)
    out = lmh.logprob_reduce(f16_tensor(x16), s, k)
    check_reduce(out, x16, sel, k, *oracle.reduce(x16, sel, k))
    assert int(out.device_error.item()) == 0
    return out


@pytest.mark.parametrize("dist,k", [("normal", 0), ("normal", 20), ("peaked", 1), ("gumbel", 128),
                                    ("gumbel", 20)])
def test_scoring_chunk_f16(dist, k):
    """256 x 248,320 f16 chunks with planted K-th ties and -inf entries."""
    seed = 5000 + 100 * ["normal", "peaked", "gumbel"].index(dist) + k
    print(f"f16 scoring chunk dist={dist} k={k} seed={seed}", flush=True)
    x, sel = synth.scoring_chunk(seed, dist, k, dtype="f16")
    _run(x, sel, k)


def test_decode_rows_f16():
    """32 x 151,936 rows of 2*N(0,1) with a +12 peak, as f16."""
    g = synth.rng(5900)
    x = synth.normal_f32(g, (32, synth.VOCAB_QWEN3), 2.0)
    x[np.arange(32), g.integers(0, synth.VOCAB_QWEN3, size=32)] += np.float32(12.0)
    x16 = x.astype(np.float16)
    sel = np.argmax(x16, axis=1).astype(np.int32)
    out = _run(x16, sel, 5)
    assert np.array_equal(out.topk_ids.cpu().numpy()[:, 0], sel)


def test_edge_rows_f16():
    """All -inf; 100 finite entries at K = 128; a constant row; -0/+0 ties; the
    largest finite f16 (65504) and subnormals (down to 2^-24); the K-th value
    tied across many blocks."""
    V = 248_320
    one, ninf = np.float16(1.0), np.float16(-np.inf)
    rows = np.full((6, V), one, dtype=np.float16)
    rows[0, :] = ninf
    rows[1, :] = ninf
    pos = synth.rng(5).choice(V, size=100, replace=False)
    rows[1, pos] = synth.normal_f32(synth.rng(6), (100,)).astype(np.float16)
    rows[3, :] = np.where(np.arange(V) % 2 == 0, np.float16(-0.0), np.float16(0.0))
    rows[3, 77_777] = one
    rows[4, :] = np.float16(-1.0)
    rows[4, ::997] = np.float16(2.0)
    sub = (np.arange(V) % 1024).astype(np.uint16)               # subnormal bit patterns 0..1023
    rows[5, :] = sub.view(np.float16)
    rows[5, 12_345] = np.float16(65504.0)
    rows[5, 200_000] = np.float16(-65504.0)
    sel = np.array([0, int(pos[0]), 5, 77_777, V - 1, 200_000], dtype=np.int32)
    out = _run(rows, sel, 128)
    ids = out.topk_ids.cpu().numpy()
    assert ids[0].tolist() == list(range(128))
    assert ids[2].tolist() == list(range(128))
    assert ids[3, 0] == 77_777 and ids[3, 1:].tolist() == list(range(127))
    assert ids[5, 0] == 12_345 and ids[5, 1] == 1023          # then the largest subnormal, lowest id


@pytest.mark.parametrize("V", [1, 65, 1000, 4097, 8192])
def test_ragged_vocab_f16(V):
    g = synth.rng(5800 + V)
    x = synth.normal_f32(g, (7, V), 2.0).astype(np.float16)
    x[:, g.integers(0, V, size=3)] = x.max()
    ld = -(-V // 8) * 8
    full = np.full((7, ld), -np.inf, dtype=np.float16)
    full[:, :V] = x
    t = f16_tensor(full)[:, :V]
    sel = g.integers(0, V, size=7).astype(np.int32)
    nb = -(-V // 64)
    for k in sorted({0, 1, min(V, 5), min(V, nb), min(V, nb + 1), V if V <= 8192 else 128}):
        if min(k, nb) * 64 > 8192:
            continue
        out = lmh.logprob_reduce(t, i32_tensor(sel), k)
        check_reduce(out, x, sel, k, *oracle.reduce(x, sel, k))


@pytest.mark.parametrize("k", [0, 20, 128])
def test_row_path_matches_split_path_f16(k):
    """256 f16 rows in one call (one workgroup per row on a 256-CU device)
    against the same rows 100 at a time (split path): bitwise equal."""
    V, R = 151_936, 256
    x, sel = synth.scoring_chunk(5700 + k, "gumbel", k, rows=R, vocab=V, dtype="f16")
    t = f16_tensor(x)
    a = lmh.logprob_reduce(t, i32_tensor(sel), k)
    parts = [lmh.logprob_reduce(t[i:i + 100], i32_tensor(sel[i:i + 100]), k) for i in range(0, R, 100)]
    torch.cuda.synchronize()
    cat = lambda f: torch.cat([getattr(p, f) for p in parts])
    assert torch.equal(a.lse.view(torch.int32), cat("lse").view(torch.int32))
    assert torch.equal(a.selected_logprob.view(torch.int32), cat("selected_logprob").view(torch.int32))
    if k > 0:
        assert torch.equal(a.topk_ids, cat("topk_ids"))
        assert torch.equal(a.topk_logprobs.view(torch.int32), cat("topk_logprobs").view(torch.int32))
    pick = np.array([0, 1, 99, 100, 255])
    sub = lmh.Reduction(a.lse[pick], a.selected_logprob[pick], a.topk_ids[pick], a.topk_logprobs[pick],
                        a.device_error)
    xs = np.ascontiguousarray(x[pick])
    check_reduce(sub, xs, sel[pick], k, *oracle.reduce(xs, sel[pick], k))


def test_f16_rejected_by_the_head():
    """f16 is a reduction input only: the head rejects it."""
    h = torch.zeros((4, 64), dtype=torch.float16, device="cuda:0")
    w = torch.zeros((100, 64), dtype=torch.float16, device="cuda:0")
    with pytest.raises(RuntimeError, match="LMH_ERR_DTYPE"):
        lmh.lmhead_gather_project(h, w, i32_tensor([0, 4]), 0)
