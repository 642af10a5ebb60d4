"""Shared helpers for the GPU parity tests (host-side conversions only)."""
import numpy as np
import torch

import synth


def dev():
    return torch.device("cuda:0")


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    """Raw bf16 bits (uint16) -> bfloat16 device tensor, bit-exact."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def i32_tensor(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def f32_tensor(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def as_f32(logits_np: np.ndarray) -> np.ndarray:
    """Host float32 values of raw-bf16 or float32 logits."""
    return synth.bf16_bits_to_f32(logits_np) if logits_np.dtype == np.uint16 else logits_np


def check_reduce(out, logits_np, sel, k, lse_ref, sel_ref, ids_ref, lp_ref, atol=1e-5):
    """Parity of a GPU reduction with the f64 oracle on the same logits:
    exact ids; lse, selected and top-K logprobs within atol; each top-K
    logprob equals float32(logit) - lse_gpu rounded once (bitwise)."""
    torch.cuda.synchronize()
    lse = out.lse.cpu().numpy()
    assert np.array_equal(np.isnan(lse), np.isnan(lse_ref))
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    fin = np.isfinite(lse_ref)
    lse_tol = np.maximum(atol, np.abs(lse_ref[fin]) * 2.0 ** -23)   # see _close_or_same_special
    assert np.all(np.abs(lse[fin] - lse_ref[fin]) <= lse_tol), np.max(np.abs(lse[fin] - lse_ref[fin]))
    x = as_f32(logits_np)
    if sel is not None:
        s = out.selected_logprob.cpu().numpy()
        _close_or_same_special(s, sel_ref, atol)
    if k:
        ids = out.topk_ids.cpu().numpy()
        lp = out.topk_logprobs.cpu().numpy()
        assert np.array_equal(ids, ids_ref), _first_diff(ids, ids_ref)
        _close_or_same_special(lp, lp_ref, atol)
        rows = np.arange(ids.shape[0])[:, None]
        want = (x[rows, ids] - lse[:, None].astype(np.float32)).astype(np.float32)
        assert np.array_equal(lp.view(np.uint32)[~np.isnan(want)], want.view(np.uint32)[~np.isnan(want)])


def _close_or_same_special(a, ref, atol):
    """|a - ref| <= atol, or one fp32 ulp of ref (2^-23 |ref|) where that is
    larger: above |ref| = 84 an fp32 result cannot be within 1e-5 of every
    exact value (half an ulp exceeds it), and the GPU's lse and logprobs are
    fp32 by definition (MTPLX PR #532, Change)."""
    a = np.asarray(a, dtype=np.float64)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(a), nan_ref)
    inf_ref = np.isinf(ref)
    assert np.array_equal(a[inf_ref], ref[inf_ref])
    m = ~nan_ref & ~inf_ref
    if m.any():
        d = np.abs(a[m] - ref[m])
        tol = np.maximum(atol, np.abs(ref[m]) * 2.0 ** -23)
        assert np.all(d <= tol), float(np.max(d - tol))


def _first_diff(a, b):
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return "equal"
    r, c = idx[0]
    return f"row {r} col {c}: gpu {a[r, c]} oracle {b[r, c]} (gpu row {a[r, :8]}, oracle {b[r, :8]})"
