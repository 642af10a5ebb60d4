"""GPU parity of lmhead_gather_project with the f64 oracle (vllm-metal
release v0.4.0, Summary and Testing; mlxcel PR #1969).

Bar: gather indices and logits_cu_seqlens bit-exact; head logits (bf16 in,
fp32 accumulate) within 2e-3 of the oracle relative to the row's max |logit|;
exact where the arithmetic is exact (small-integer inputs, one-hot rows);
selective rows bitwise equal to the same rows of the full projection, and
the weight-streaming and tiled kernels bitwise equal to each other."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_bits, bf16_tensor, f32_tensor, i32_tensor

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _check_rows(proj, cu, nd, T, ex=None):
    st, idx, lcu = oracle.rows(cu, nd, T, ex)
    assert st == oracle.OK
    torch.cuda.synchronize()
    assert np.array_equal(proj.gather_indices.cpu().numpy(), idx)
    assert np.array_equal(proj.logits_cu_seqlens.cpu().numpy(), lcu)
    assert int(proj.device_error.item()) == 0
    return idx


def _close(z, z_ref, tol=TOL):
    scale = np.abs(z_ref).max(axis=1, keepdims=True)
    err = np.abs(z.astype(np.float64) - z_ref)
    assert np.all(err <= tol * scale), float((err / scale).max())


def test_tiny_fp32_batch():
    d = synth.tiny_batch(1000)
    T = d["hidden"].shape[0]
    p = lmh.lmhead_gather_project(f32_tensor(d["hidden"]), f32_tensor(d["weight"]),
                                  i32_tensor(d["cu_seqlens"]), d["num_decode"])
    idx = _check_rows(p, d["cu_seqlens"], d["num_decode"], T)
    assert idx.tolist() == [0, 1, 6, 13, 22]
    _close(p.logits.cpu().numpy(), oracle.head(d["hidden"], d["weight"], idx), 1e-5)


@pytest.mark.parametrize("variant", [lmh.LMH_HEAD_STREAM, lmh.LMH_HEAD_TILED])
@pytest.mark.parametrize("H", [64, 96, 4096])
def test_small_integers_exact(variant, H):
    """bf16 entries in {-4..4}: every partial sum is an exact fp32 integer, so
    the MFMA result must equal the oracle bit for bit."""
    T, V = 50, 1000 + 17
    hid = synth.small_int_bf16(11, (T, H))
    w = synth.small_int_bf16(12, (V, H))
    cu = synth.packed_cu_seqlens(3, [7, 9, 1, 30])
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 3, variant=variant)
    idx = _check_rows(p, cu, 3, T)
    assert np.array_equal(p.logits.cpu().numpy().astype(np.float64), oracle.head(hid, w, idx))


def test_one_hot_rows_read_weight_columns():
    H, V = 128, 3000
    cols = [0, 1, 63, 64, 127, 5]
    hid = np.zeros((len(cols), H), dtype=np.uint16)
    for t, j in enumerate(cols):
        hid[t, j] = 0x3F80                                   # 1.0
    w = synth.normal_bf16(synth.rng(13), (V, H))
    ex = np.arange(len(cols), dtype=np.int32)
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, len(cols)]), 0,
                                  logits_indices=i32_tensor(ex))
    z = p.logits.cpu().numpy()
    wf = synth.bf16_bits_to_f32(w)
    for t, j in enumerate(cols):
        assert np.array_equal(z[t], wf[:, j])


@pytest.mark.parametrize("R", [1, 17, 64, 65, 130])
@pytest.mark.parametrize("V", [1000, 1001, 4096])
def test_random_bf16_shapes(R, V):
    """Ragged vocab tails, partial row tiles, both kernels (R <= 64 streams)."""
    g = synth.rng(R * 7 + V)
    H, T = 256, 300
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = g.integers(0, T, size=R).astype(np.int32)
    cu = np.array([0, T], dtype=np.int32)
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 0,
                                  logits_indices=i32_tensor(ex))
    idx = _check_rows(p, cu, 0, T, ex)
    _close(p.logits.cpu().numpy(), oracle.head(hid, w, idx))


def test_bf16_output_is_rne_of_fp32():
    g = synth.rng(14)
    hid = synth.normal_bf16(g, (40, 512))
    w = synth.normal_bf16(g, (5000, 512), 512 ** -0.5)
    cu = synth.packed_cu_seqlens(40, [])
    args = (bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 40)
    f = lmh.lmhead_gather_project(*args).logits
    b = lmh.lmhead_gather_project(*args, out_dtype=torch.bfloat16).logits
    assert np.array_equal(bf16_bits(b), synth.f32_to_bf16_bits(f.cpu().numpy()))


@pytest.mark.parametrize("H", [96, 512])
def test_bf16_output_is_rne_of_fp32_tiled(H):
    """The same for row counts the tiled kernels take (64-wide k stages when
    the hidden size is a multiple of 128, 32-wide otherwise), with a partial
    last row tile and a partial vocabulary tile."""
    g = synth.rng(15 + H)
    T, V, R = 400, 3000, 300
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    cu = np.array([0, T], dtype=np.int32)
    ex = g.integers(0, T, size=R).astype(np.int32)
    args = (bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 0)
    f = lmh.lmhead_gather_project(*args, logits_indices=i32_tensor(ex)).logits
    b = lmh.lmhead_gather_project(*args, logits_indices=i32_tensor(ex), out_dtype=torch.bfloat16).logits
    assert np.array_equal(bf16_bits(b), synth.f32_to_bf16_bits(f.cpu().numpy()))
    _close(f.cpu().numpy(), oracle.head(hid, w, ex))


def test_invalid_rows_are_nan_and_flagged():
    g = synth.rng(15)
    hid = synth.normal_bf16(g, (10, 64))
    w = synth.normal_bf16(g, (300, 64))
    ex = np.array([0, 10, -3, 9], dtype=np.int32)
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, 10]), 0,
                                  logits_indices=i32_tensor(ex))
    torch.cuda.synchronize()
    z = p.logits.cpu().numpy()
    assert np.all(np.isfinite(z[[0, 3]])) and np.all(np.isnan(z[[1, 2]]))
    assert p.gather_indices.cpu().numpy().tolist() == [0, -1, -1, 9]
    assert int(p.device_error.item()) & lmh.LMH_DEVERR_INDEX
    # a decode segment of two tokens is a layout error
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, 2, 5]), 1)
    torch.cuda.synchronize()
    assert int(p.device_error.item()) & lmh.LMH_DEVERR_LAYOUT
    assert np.all(np.isnan(p.logits.cpu().numpy()[0]))


@pytest.mark.parametrize("H", [64, 128])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_invalid_rows_are_nan_tiled(H, out):
    """Row counts the tiled kernels take (64-wide k stages at H = 128): rows
    with an out-of-range index come out NaN and flagged, the others match
    the oracle."""
    g = synth.rng(16 + H)
    T, V, R = 50, 700, 100
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = g.integers(0, T, size=R).astype(np.int32)
    bad = np.array([3, 50, 99])
    ex[bad] = [T, -1, T + 7]
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, T]), 0,
                                  logits_indices=i32_tensor(ex), out_dtype=out)
    torch.cuda.synchronize()
    z = p.logits.float().cpu().numpy()
    good = np.setdiff1d(np.arange(R), bad)
    assert np.all(np.isnan(z[bad])) and np.all(np.isfinite(z[good]))
    assert int(p.device_error.item()) & lmh.LMH_DEVERR_INDEX
    if out == torch.float32:
        _close(z[good], oracle.head(hid, w, ex[good]))


@pytest.mark.parametrize("mode,s", [(lmh.LMH_SCALE_NONE, 1.0), (lmh.LMH_SCALE_MUL, 0.3), (lmh.LMH_SCALE_DIV, 6.0)])
def test_tiled_walk_ragged(mode, s):
    """600 rows x (151,936 - 37) vocabulary at hidden 256: more than four row
    x vocab tiles per CU, so each workgroup walks several tiles and loads
    the next tile's first stages before its epilogue; the last row tile and
    the last vocab tile are partial and four rows have no source. Those rows
    are NaN and flagged; 12 rows (the partial row tile included) match the
    scaled oracle at every column; 40 rows equal, bit for bit, the same rows
    projected by the weight-streaming kernel; scaled logits are one fp32
    multiply or IEEE division of the unscaled ones."""
    g = synth.rng(40 + mode)
    T, H, V, R = 700, 256, 151_936 - 37, 600
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = g.integers(0, T, size=R).astype(np.int32)
    bad = np.array([5, 300, 513, 599])
    ex[bad] = [T, -2, T + 1, -1]
    head = lmh.HeadSpec(bf16_tensor(w), mode, s)
    hid_t, cu_t = bf16_tensor(hid), i32_tensor([0, T])
    p = lmh.lmhead_gather_project_ex(hid_t, head, cu_t, 0, logits_indices=i32_tensor(ex),
                                     variant=lmh.LMH_HEAD_TILED)
    print(f"tiled walk {R} x {V} x {H} mode {mode}", flush=True)
    torch.cuda.synchronize()
    z = p.logits.cpu().numpy()
    good = np.setdiff1d(np.arange(R), bad)
    assert np.all(np.isnan(z[bad])) and np.all(np.isfinite(z[good]))
    assert int(p.device_error.item()) & lmh.LMH_DEVERR_INDEX
    rows = np.concatenate([g.choice(good[good < 512], size=8, replace=False), good[good >= 512][-4:]])
    _close(z[rows], oracle.head(hid, w, ex[rows], scale_mode=mode, scale=s))
    sel = g.choice(good, size=40, replace=False)
    q = lmh.lmhead_gather_project_ex(hid_t, head, cu_t, 0, logits_indices=i32_tensor(ex[sel]),
                                     variant=lmh.LMH_HEAD_STREAM)
    torch.cuda.synchronize()
    assert np.array_equal(q.logits.cpu().numpy().view(np.uint32), z[sel].view(np.uint32))
    if mode != lmh.LMH_SCALE_NONE:
        u = lmh.lmhead_gather_project_ex(hid_t, lmh.HeadSpec(head.weight), cu_t, 0,
                                         logits_indices=i32_tensor(ex), variant=lmh.LMH_HEAD_TILED)
        zu = u.logits.cpu().numpy()[good].astype(np.float32)
        want = zu * np.float32(s) if mode == lmh.LMH_SCALE_MUL else zu / np.float32(s)
        assert np.array_equal(z[good].view(np.uint32), want.view(np.uint32))


@pytest.fixture(scope="module")
def qwen_batch():
    return synth.selective_head_batch(4000)


def test_selective_head_qwen_shape(qwen_batch):
    """40 prefill segments x 2048 tokens, hidden 1024, vocab 151,936: gather the
    40 last rows; every logit of every row against the oracle."""
    d = qwen_batch
    T = d["hidden"].shape[0]
    hid, w = bf16_tensor(d["hidden"]), bf16_tensor(d["weight"])
    p = lmh.lmhead_gather_project(hid, w, i32_tensor(d["cu_seqlens"]), 0)
    idx = _check_rows(p, d["cu_seqlens"], 0, T)
    assert np.array_equal(idx, 2047 + 2048 * np.arange(40))
    print("oracle head: 40 x 151936 x 1024", flush=True)
    _close(p.logits.cpu().numpy(), oracle.head(d["hidden"], d["weight"], idx))


def test_full_projection_rows_against_oracle(qwen_batch):
    """The 2048-row projection of segment 0 (the large-row tiled kernel): 32
    seeded rows, every logit, against the oracle."""
    d = qwen_batch
    hid, w = bf16_tensor(d["hidden"]), bf16_tensor(d["weight"])
    full = lmh.lmhead_gather_project(hid, w, i32_tensor(d["cu_seqlens"]), 0,
                                     logits_indices=i32_tensor(np.arange(2048))).logits
    rows = np.sort(synth.rng(18).choice(2048, size=32, replace=False)).astype(np.int32)
    torch.cuda.synchronize()
    print("oracle head: 32 x 151936 x 1024", flush=True)
    _close(full.cpu().numpy()[rows], oracle.head(d["hidden"], d["weight"], rows))


def test_selective_equals_full_projection_bitwise(qwen_batch):
    """The selective rows equal the same rows of the full 2048-row projection
    of segment 0, bit for bit; the row one off does not (the control)."""
    d = qwen_batch
    hid, w = bf16_tensor(d["hidden"]), bf16_tensor(d["weight"])
    cu = i32_tensor(d["cu_seqlens"])
    full = lmh.lmhead_gather_project(hid, w, cu, 0,
                                     logits_indices=i32_tensor(np.arange(2048))).logits
    sel = lmh.lmhead_gather_project(hid, w, cu, 0).logits
    tiled = lmh.lmhead_gather_project(hid, w, cu, 0, variant=lmh.LMH_HEAD_TILED).logits
    torch.cuda.synchronize()
    assert torch.equal(full[2047].view(torch.int32), sel[0].view(torch.int32))
    assert torch.equal(tiled.view(torch.int32), sel.view(torch.int32))
    assert not torch.equal(full[2046], sel[0])
    # a mid-segment row through the streaming kernel matches the full projection
    mid = lmh.lmhead_gather_project(hid, w, cu, 0, logits_indices=i32_tensor([1000, 5, 2047]),
                                    variant=lmh.LMH_HEAD_STREAM).logits
    torch.cuda.synchronize()
    assert torch.equal(mid.view(torch.int32), full[[1000, 5, 2047]].view(torch.int32))


def test_pure_decode_identity():
    """Pure decode: every row is sampled, in order (vllm-metal release: pure
    decode is unchanged)."""
    g = synth.rng(17)
    hid = synth.normal_bf16(g, (33, 128))
    w = synth.normal_bf16(g, (2000, 128), 128 ** -0.5)
    cu = synth.packed_cu_seqlens(33, [])
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 33)
    full = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 0,
                                     logits_indices=i32_tensor(np.arange(33))).logits
    torch.cuda.synchronize()
    assert np.array_equal(p.gather_indices.cpu().numpy(), np.arange(33))
    assert torch.equal(p.logits.view(torch.int32), full.view(torch.int32))


@pytest.mark.parametrize("weights", ["bf16", "q4"])
@pytest.mark.parametrize("mode,s", [(lmh.LMH_SCALE_NONE, 1.0), (lmh.LMH_SCALE_MUL, 0.125), (lmh.LMH_SCALE_DIV, 3.0)])
@pytest.mark.parametrize("odt,pad", [("f32", 0), ("f32", 4), ("f32", 1), ("bf16", 0), ("bf16", 8), ("bf16", 4)])
def test_stream_row_segment_stores(weights, mode, s, odt, pad):
    """The streaming kernels' logits go out as whole row segments through LDS
    when the vocabulary and the row pitch are multiples of 4 fp32 or 8 bf16
    logits (fp32 pad 0, 4; bf16 pad 0, 8; the others take the element
    stores): bitwise the tiled kernel's fp32 logits (bf16: their
    round-to-nearest-even), NaN on the rows without a source, the pitch
    padding untouched, with and without output scaling; V = 5000 leaves the
    last workgroup's columns partly past the vocabulary."""
    g = synth.rng(4300 + pad + 7 * mode)
    H, V, T, R = 1024, 5000, 200, 40
    hid = synth.normal_bf16(g, (T, H))
    if weights == "bf16":
        wt = bf16_tensor(synth.normal_bf16(g, (V, H), H ** -0.5))
    else:
        d = synth.quantized_head(4301, V, H, 4, 64)
        wt = lmh.QuantizedWeight(torch.from_numpy(d["q"].view(np.int32)).cuda(), bf16_tensor(d["scales"]),
                                 bf16_tensor(d["biases"]), 4, 64)
    head = lmh.HeadSpec(wt, mode, s)
    ex = g.integers(0, T, size=R).astype(np.int32)
    bad = np.array([2, 17, 39])
    ex[bad] = T + 5                                            # no source: NaN rows
    args = (bf16_tensor(hid), head, i32_tensor([0, T]), 0)
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    out = torch.full((R, V + pad), 7.0, dtype=tdt, device="cuda")
    print(f"stream row segments {weights} mode {mode} {odt} pad {pad}", flush=True)
    st = lmh.lmhead_gather_project_ex(*args, logits_indices=i32_tensor(ex), logits=out[:, :V],
                                      variant=lmh.LMH_HEAD_STREAM)
    ti = lmh.lmhead_gather_project_ex(*args, logits_indices=i32_tensor(ex), variant=lmh.LMH_HEAD_TILED)
    torch.cuda.synchronize()
    b = ti.logits.cpu().numpy()
    good = np.setdiff1d(np.arange(R), bad)
    if odt == "f32":
        a = out[:, :V].cpu().numpy()
        assert np.all(np.isnan(a[bad]))
        assert np.array_equal(a[good].view(np.uint32), b[good].view(np.uint32))
    else:
        bits = bf16_bits(out[:, :V])
        assert np.all(((bits[bad] & 0x7F80) == 0x7F80) & ((bits[bad] & 0x7F) != 0))   # NaN
        assert np.array_equal(bits[good], synth.f32_to_bf16_bits(b[good]))
    assert int(st.device_error.item()) & lmh.LMH_DEVERR_INDEX
    if pad:
        assert torch.all(out[:, V:] == 7.0)


@pytest.mark.parametrize("H", [128, 96])
@pytest.mark.parametrize("pad", [0, 1, 3, 9])
def test_tiled_bf16_logits_pitches(H, pad):
    """bf16 logits of the tiled kernels (64-wide stages at H = 128, 32-wide at
    96) go out four per 8-byte store when the row pitch is a multiple of 4
    (V + pad = 3000, 3008) and one by one otherwise (2999, 3002): the
    round-to-nearest-even of the fp32 logits either way, the pitch padding
    untouched; V = 2999 leaves a last group of three columns."""
    g = synth.rng(4500 + H + pad)
    T, V, R = 300, 2999, 270
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = g.integers(0, T, size=R).astype(np.int32)
    args = (bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, T]), 0)
    print(f"tiled bf16 logits H={H} pad={pad}", flush=True)
    f = lmh.lmhead_gather_project(*args, logits_indices=i32_tensor(ex), variant=lmh.LMH_HEAD_TILED).logits
    out = torch.full((R, V + pad), 3.0, dtype=torch.bfloat16, device="cuda")
    lmh.lmhead_gather_project(*args, logits_indices=i32_tensor(ex), logits=out[:, :V], variant=lmh.LMH_HEAD_TILED)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out[:, :V]), synth.f32_to_bf16_bits(f.cpu().numpy()))
    if pad:
        assert torch.all(out[:, V:] == 3.0)
