"""logprob_reduce_noalloc (the reduction for callers that cannot allocate)
against logprob_reduce, through the C ABI: two calls in a row on the static
scratch, the second on a smaller input, each bitwise equal to logprob_reduce
on a workspace of its own (the same kernels run; only the scratch differs)."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import top_reduction_amd as lmh
from helpers import bf16_tensor, check_reduce, i32_tensor

import oracle

pytestmark = pytest.mark.gpu


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _outs(R, k, dev):
    return (torch.full((R,), 7.0, device=dev), torch.full((R,), 7.0, device=dev),
            torch.full((R, k), 7, dtype=torch.int32, device=dev), torch.full((R, k), 7.0, device=dev),
            torch.zeros(1, dtype=torch.int32, device=dev))


def _call(L, fn, logits, sel, k, o, ws=None):
    R, V = logits.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dt = lmh.LMH_BF16 if logits.dtype == torch.bfloat16 else lmh.LMH_F32
    args = [_vp(logits), dt, R, V, logits.stride(0), _vp(sel), k, _vp(o[0]), _vp(o[1]),
            _vp(o[2]) if k else None, _vp(o[3]) if k else None]
    if ws is not None:
        args += [_vp(ws), ws.numel()]
    args += [_vp(o[4]), stream]
    return fn(*args)


def _same(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                           y.view(torch.int32) if y.dtype == torch.float32 else y)


def test_noalloc_matches_logprob_reduce():
    L = lmh.lib()
    dev = torch.device("cuda:0")
    # call 1: 32 decode rows x 151,936; call 2: a smaller input, 5 rows x
    # 40,000 with K = 3 (both take the single-launch path, which uses the
    # scratch and its per-row counters)
    bits1, sel1 = synth.decode_logits(8100, sel_mode="uniform")
    g = synth.rng(8101)
    bits2 = synth.normal_bf16(g, (5, 40000), 2.0)
    sel2 = g.integers(0, 40000, size=5).astype(np.int32)
    cases = [(bf16_tensor(bits1), i32_tensor(sel1), 5, bits1, sel1),
             (bf16_tensor(bits2), i32_tensor(sel2), 3, bits2, sel2)]
    got = []
    for logits, sel, k, bits, sel_np in cases:
        R = logits.shape[0]
        assert not lmh.reduce_row_path(R, logits.shape[1], k)
        o = _outs(R, k, dev)
        assert _call(L, L.logprob_reduce_noalloc, logits, sel, k, o) == 0
        got.append((o, logits, sel, k, bits, sel_np))
    torch.cuda.synchronize()
    for o, logits, sel, k, bits, sel_np in got:
        R, V = logits.shape
        ref = _outs(R, k, dev)
        ws = torch.empty(L.logprob_reduce_workspace_size(R, V, k), dtype=torch.uint8, device=dev)
        assert _call(L, L.logprob_reduce, logits, sel, k, ref, ws) == 0
        torch.cuda.synchronize()
        _same(o, ref)
        assert int(o[4].item()) == 0
        # and the oracle, to the reduction's bar
        red = lmh.Reduction(o[0], o[1], o[2], o[3], o[4])
        check_reduce(red, bits, sel_np, k, *oracle.reduce(bits, sel_np, k))


def test_noalloc_rejects_oversized_shape():
    L = lmh.lib()
    dev = torch.device("cuda:0")
    logits = torch.empty((600, 248320), dtype=torch.bfloat16, device=dev)
    o = _outs(600, 1, dev)
    assert _call(L, L.logprob_reduce_noalloc, logits, None, 0, o) == 6   # LMH_ERR_WORKSPACE
