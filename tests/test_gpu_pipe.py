"""GPU parity of the k-pipelined weight-streaming head (LMH_HEAD_PIPE) with
the f64 oracle and with the other bf16 head kernels (vllm-metal release
v0.4.0, Summary and Testing; mlxcel PR #1969: a gathered row's logits equal
the full projection's).

The pipelined kernel chains the hidden dimension across the 16 waves of a
workgroup and passes the partial sums between them, so each logit sees the
same MFMA sequence as in the streaming and tiled kernels: the three must agree
bit for bit. Shapes cover every hidden size it takes (512..2048), partial row
tiles (R not a multiple of 16), a ragged vocabulary tail (V not a multiple of
16), fewer tiles than workgroups, row pitches, bf16 output, output scaling and
rows without a source."""
import numpy as np
import pytest
import torch

import oracle
import synth
import top_reduction_amd as lmh
from helpers import bf16_bits, bf16_tensor, i32_tensor

pytestmark = pytest.mark.gpu

TOL = 2e-3
PIPE, STREAM, TILED = lmh.LMH_HEAD_PIPE, lmh.LMH_HEAD_STREAM, lmh.LMH_HEAD_TILED


def _bits(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int32).cpu().numpy()


def _close(z, z_ref, tol=TOL):
    scale = np.abs(z_ref).max(axis=1, keepdims=True)
    err = np.abs(z.astype(np.float64) - z_ref)
    assert np.all(err <= tol * scale), float((err / scale).max())


@pytest.mark.parametrize("H", [512, 1024, 1536, 2048])
@pytest.mark.parametrize("R", [1, 17, 40, 64])
def test_small_integers_exact(H, R):
    """bf16 entries in {-4..4}: exact fp32 sums in any order, so the pipelined
    kernel must equal the oracle bit for bit."""
    T, V = 70, 1000 + 9
    hid = synth.small_int_bf16(100 + R, (T, H))
    w = synth.small_int_bf16(200 + R, (V, H))
    ex = synth.rng(300 + R).integers(0, T, size=R).astype(np.int32)
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, T]), 0,
                                  logits_indices=i32_tensor(ex), variant=PIPE)
    torch.cuda.synchronize()
    assert int(p.device_error.item()) == 0
    assert np.array_equal(p.logits.cpu().numpy().astype(np.float64), oracle.head(hid, w, ex))


@pytest.mark.parametrize("H,R,V", [(1024, 40, 20011), (512, 5, 4097), (2048, 64, 9000),
                                   (1536, 33, 16), (1024, 16, 100), (2048, 48, 50257),
                                   (1024, 40, 4100), (512, 64, 20012)])
def test_bitwise_equal_to_stream_and_tiled(H, R, V):
    """Random bf16 rows: the pipelined, streaming and tiled kernels give the
    same bits; all within the head tolerance of the f64 oracle. V = 16 and
    V = 100 give fewer 16-row tiles than workgroups; with fp32 logits and V a
    multiple of 4 (9000, 100, 4100, 20012) tile pairs are stored as whole
    rows, and runs of one or two tiles that start or end inside a pair store
    their half alone (4100: a last tile of four columns)."""
    g = synth.rng(H + 7 * R + V)
    T = 300
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = g.integers(0, T, size=R).astype(np.int32)
    args = (bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, T]), 0)
    outs = [lmh.lmhead_gather_project(*args, logits_indices=i32_tensor(ex), variant=v).logits
            for v in (PIPE, STREAM, TILED)]
    b = [_bits(o) for o in outs]
    assert np.array_equal(b[0], b[1]) and np.array_equal(b[0], b[2])
    cols = np.sort(g.choice(V, size=min(V, 2048), replace=False))
    _close(outs[0].cpu().numpy()[:, cols], oracle.head(hid, np.ascontiguousarray(w[cols]), ex))


def test_auto_takes_the_pipeline_and_matches_full_projection():
    """Sampled mode with H = 1024 and 16 < R <= 64 runs the pipelined kernel;
    its rows equal the same rows of a full (tiled) projection bit for bit."""
    g = synth.rng(41)
    H, V = 1024, 30011
    lens = [300, 1, 77, 512, 2, 9, 40, 3, 5, 6, 7, 8, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20]
    cu = synth.packed_cu_seqlens(0, lens)
    T = int(cu[-1])
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    a = (bf16_tensor(hid), bf16_tensor(w), i32_tensor(cu), 0)
    auto = lmh.lmhead_gather_project(*a).logits
    pipe = lmh.lmhead_gather_project(*a, variant=PIPE).logits
    full = lmh.lmhead_gather_project(*a, logits_indices=i32_tensor(np.arange(T)), variant=TILED).logits
    rows = cu[1:] - 1
    assert np.array_equal(_bits(auto), _bits(pipe))
    assert np.array_equal(_bits(pipe), _bits(full)[rows])


def test_row_pitches_and_bf16_output():
    """Hidden, weight and logits with row pitches wider than their rows; bf16
    logits are the round-to-nearest-even of the fp32 ones."""
    g = synth.rng(42)
    H, V, T, R = 1024, 5003, 90, 23
    hid_big = synth.normal_bf16(g, (T, H + 72))
    w_big = synth.normal_bf16(g, (V, H + 40), H ** -0.5)
    ex = g.integers(0, T, size=R).astype(np.int32)
    hid = bf16_tensor(hid_big)[:, :H]
    w = bf16_tensor(w_big)[:, :H]
    out = torch.full((R, V + 13), 7.0, dtype=torch.float32, device=hid.device)
    a = (hid, w, i32_tensor([0, T]), 0)
    lmh.lmhead_gather_project(*a, logits_indices=i32_tensor(ex), logits=out[:, :V], variant=PIPE)
    ref = lmh.lmhead_gather_project(*a, logits_indices=i32_tensor(ex), variant=STREAM).logits
    assert np.array_equal(_bits(out[:, :V]), _bits(ref))
    assert torch.all(out[:, V:] == 7.0)                       # the pitch padding is untouched
    b = lmh.lmhead_gather_project(*a, logits_indices=i32_tensor(ex), out_dtype=torch.bfloat16,
                                  variant=PIPE).logits
    assert np.array_equal(bf16_bits(b), synth.f32_to_bf16_bits(ref.cpu().numpy()))


def test_rows_without_source_are_nan():
    g = synth.rng(43)
    H, V, T = 512, 3000, 12
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = np.array([0, T, -1, 11, 5], dtype=np.int32)
    p = lmh.lmhead_gather_project(bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, T]), 0,
                                  logits_indices=i32_tensor(ex), variant=PIPE)
    torch.cuda.synchronize()
    z = p.logits.cpu().numpy()
    assert np.all(np.isnan(z[[1, 2]])) and np.all(np.isfinite(z[[0, 3, 4]]))
    assert int(p.device_error.item()) & lmh.LMH_DEVERR_INDEX
    _close(z[[0, 3, 4]], oracle.head(hid, w, ex[[0, 3, 4]]))


@pytest.mark.parametrize("mode,scale", [(lmh.LMH_SCALE_MUL, 0.0625), (lmh.LMH_SCALE_DIV, 7.0)])
def test_output_scaling_matches_stream(mode, scale):
    """The multiply and divide head scalings give the same bits as in the
    weight-streaming kernel (one fp32 operation on the same fp32 logit)."""
    g = synth.rng(44)
    H, V, T, R = 2048, 7001, 40, 40
    hid = bf16_tensor(synth.normal_bf16(g, (T, H)))
    w = bf16_tensor(synth.normal_bf16(g, (V, H), H ** -0.5))
    head = lmh.HeadSpec(w, scale_mode=mode, scale=scale)
    cu = i32_tensor(synth.packed_cu_seqlens(R, []))
    a = lmh.lmhead_gather_project_ex(hid, head, cu, R, variant=PIPE).logits
    b = lmh.lmhead_gather_project_ex(hid, head, cu, R, variant=STREAM).logits
    plain = lmh.lmhead_gather_project(hid, w, cu, R, variant=STREAM).logits
    assert np.array_equal(_bits(a), _bits(b))
    # the correctly rounded fp32 product / quotient: the f64 operation on two
    # fp32 values, rounded once to fp32 (f64 carries enough bits that the
    # double rounding is exact for * and /)
    x = plain.cpu().numpy().astype(np.float64)
    want = (x * scale if mode == lmh.LMH_SCALE_MUL else x / scale).astype(np.float32)
    assert np.array_equal(_bits(a), want.view(np.int32))


@pytest.mark.parametrize("H,R", [(256, 8), (4096, 8), (1024, 65), (1032, 8)])
def test_rejects_shapes_outside_its_range(H, R):
    g = synth.rng(45)
    hid = bf16_tensor(synth.normal_bf16(g, (R, H)))
    w = bf16_tensor(synth.normal_bf16(g, (64, H)))
    with pytest.raises(RuntimeError, match="LMH_ERR_SHAPE"):
        lmh.lmhead_gather_project(hid, w, i32_tensor([0, R]), 0,
                                  logits_indices=i32_tensor(np.arange(R)), variant=PIPE)


@pytest.mark.parametrize("V", [9000, 4104, 64, 5000])
def test_bf16_logits_grouped_rows(V):
    """bf16 logits with a vocabulary that is a multiple of 8 leave in groups
    of four tiles as whole 128-byte rows (5000 = 8 * 625 too; runs that start
    or end inside a group store their part alone): the round-to-nearest-even
    of the fp32 logits, NaN on rows without a source, the pitch padding
    untouched."""
    g = synth.rng(4400 + V)
    H, T, R = 1024, 120, 40
    hid = synth.normal_bf16(g, (T, H))
    w = synth.normal_bf16(g, (V, H), H ** -0.5)
    ex = g.integers(0, T, size=R).astype(np.int32)
    ex[[5, 33]] = T + 3                                      # no source
    a = (bf16_tensor(hid), bf16_tensor(w), i32_tensor([0, T]), 0)
    print(f"pipe bf16 grouped rows V={V}", flush=True)
    ref = lmh.lmhead_gather_project(*a, logits_indices=i32_tensor(ex), variant=PIPE).logits
    out = torch.full((R, V + 8), 7.0, dtype=torch.bfloat16, device="cuda")
    lmh.lmhead_gather_project(*a, logits_indices=i32_tensor(ex), logits=out[:, :V], variant=PIPE)
    torch.cuda.synchronize()
    z = ref.cpu().numpy()
    bits = bf16_bits(out[:, :V])
    good = np.setdiff1d(np.arange(R), [5, 33])
    assert np.all(np.isnan(z[[5, 33]]))
    assert np.all(((bits[[5, 33]] & 0x7F80) == 0x7F80) & ((bits[[5, 33]] & 0x7F) != 0))   # NaN
    assert np.array_equal(bits[good], synth.f32_to_bf16_bits(z[good]))
    assert torch.all(out[:, V:] == 7.0)
