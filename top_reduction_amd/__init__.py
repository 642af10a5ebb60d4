"""Selective LM head and on-device logprob reduction for AMD MI355X (gfx950).

A thin ctypes binding over ``liblmhead.so`` (C ABI in ``include/lmhead.h``).
This module only marshals arguments: tensors become device pointers and row
pitches, outputs and workspaces are allocated with torch, and every call is
enqueued on torch's current HIP stream. Every step of the computation runs in
the library's HIP kernels; there is no fallback, and a missing library raises.

Entry points (same names as the C ABI):
  lmhead_gather_project  gather the sampled rows of a packed batch and project
                         only those through the head
  logprob_reduce         per-row logsumexp, selected logprob, exact top-K
  lmhead_logprobs        both, fused and chunked
  lmhead_gather_project_q, lmhead_logprobs_q
                         the same with an affine group-quantised head
                         (QuantizedWeight: 4- or 8-bit codes, bf16 scale and
                         bias per group)
  lmhead_gather_project_ex, lmhead_logprobs_ex
                         the same with a HeadSpec (dense or quantised weights
                         plus output scaling)
  lmhead_selfcheck       bit-exact check of the selective rows against a
                         head's own full output
  lmhead_apply_bitmask   token bitmask on the compacted logits rows of each
                         segment, in place
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch

from ._abi import (LIB_PATH, LMH_BF16, LMH_DEVERR_INDEX, LMH_DEVERR_LAYOUT, LMH_F16, LMH_F32,  # noqa: F401
                   LMH_HEAD_AUTO, LMH_HEAD_PIPE, LMH_HEAD_STREAM, LMH_HEAD_TILED, LMH_K_FULL,
                   LMH_SCALE_DIV, LMH_SCALE_MUL, LMH_SCALE_NONE, STATUS, LmhError, LmhHead)
from ._abi import load as _load

_lib = None


def lib():
    """Load liblmhead.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise LmhError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t: torch.Tensor) -> int:
    """lmh_dtype of a tensor (the library rejects f16 everywhere but in the
    reduction's logits)."""
    if t.dtype == torch.bfloat16:
        return LMH_BF16
    if t.dtype == torch.float32:
        return LMH_F32
    if t.dtype == torch.float16:
        return LMH_F16
    raise TypeError(f"unsupported dtype {t.dtype} (bf16, f16 or fp32)")


def _matrix(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.shape[0], t.shape[1], t.stride(0)


def _i32(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 device tensor")
    return t


def _topk_out(R: int, V: int, k: int, dev):
    """Top-K outputs: ids [R, k] and logprobs [R, k]; for k = LMH_K_FULL no
    ids and every token's logprob [R, V]."""
    if k == LMH_K_FULL:
        return (torch.empty((R, 0), dtype=torch.int32, device=dev),
                torch.empty((R, V), dtype=torch.float32, device=dev))
    return (torch.empty((R, max(k, 0)), dtype=torch.int32, device=dev),
            torch.empty((R, max(k, 0)), dtype=torch.float32, device=dev))


def _topk_ptrs(k: int, ids: torch.Tensor, lps: torch.Tensor):
    if k == LMH_K_FULL:
        return None, _ptr(lps)
    return (_ptr(ids), _ptr(lps)) if k else (None, None)


def workspace(nbytes: int, device) -> torch.Tensor:
    """A 256-byte-aligned byte buffer (torch's caching allocator aligns more)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Projection(NamedTuple):
    logits: torch.Tensor
    logits_cu_seqlens: torch.Tensor
    gather_indices: torch.Tensor
    device_error: torch.Tensor


class QuantizedWeight(NamedTuple):
    """An affine group-quantised head: weight[v][k] = scales[v][g] * code +
    biases[v][g], g = k // group_size, with the `bits`-bit codes (4 or 8) of
    row v packed little-endian in the 32-bit words q[v] (int32 storage of the
    uint32 words). scales and biases are bfloat16 [vocab, groups] with one
    row stride."""
    q: torch.Tensor
    scales: torch.Tensor
    biases: torch.Tensor
    bits: int
    group_size: int


def _dense_weight_args(weight: torch.Tensor, H: int):
    V, H2, wld = _matrix(weight, "weight")
    if H2 != H:
        raise ValueError("hidden and weight widths differ")
    return V, [_ptr(weight), _dt(weight), V, wld]


def _quant_weight_args(w: QuantizedWeight, H: int):
    V, words, qld = _matrix(w.q, "q")
    if w.q.dtype != torch.int32:
        raise ValueError("q must hold the uint32 code words as int32")
    Vs, G, sld = _matrix(w.scales, "scales")
    Vb, Gb, bld = _matrix(w.biases, "biases")
    if w.scales.dtype != torch.bfloat16 or w.biases.dtype != torch.bfloat16:
        raise ValueError("scales and biases must be bfloat16")
    if (Vs, G, sld) != (Vb, Gb, bld) or Vs != V:
        raise ValueError("scales and biases must share shape and row stride, one row per token")
    if words * 32 < H * int(w.bits) or G * int(w.group_size) < H:
        raise ValueError("q, scales and biases do not cover the hidden width")
    return V, [_ptr(w.q), qld, _ptr(w.scales), _ptr(w.biases), sld, int(w.bits), int(w.group_size), V]


def _project(fn_auto, fn_debug, name, hidden, weight_args, V, cu_seqlens, num_decode,
             logits_indices, out_dtype, logits, variant, device_error) -> Projection:
    T, H, hld = _matrix(hidden, "hidden")
    cu = _i32(cu_seqlens, "cu_seqlens")
    ex = _i32(logits_indices, "logits_indices")
    S = cu.shape[0] - 1
    R = ex.shape[0] if ex is not None else S
    dev = hidden.device
    if logits is None:
        logits = torch.empty((R, V), dtype=out_dtype, device=dev)
    _, _, old = _matrix(logits, "logits") if R > 0 else (0, 0, V)
    lcu = torch.empty(S + 1, dtype=torch.int32, device=dev)
    gidx = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
    err = device_error if device_error is not None else torch.zeros(1, dtype=torch.int32, device=dev)
    args = [_ptr(hidden), _dt(hidden), T, H, hld, *weight_args,
            _ptr(cu), S, int(num_decode), _ptr(ex), R if ex is not None else 0,
            _ptr(logits), _dt(logits), old, _ptr(lcu), _ptr(gidx), _ptr(err), _stream()]
    st = fn_auto(*args) if variant == LMH_HEAD_AUTO else fn_debug(*args, int(variant))
    _check(st, name)
    return Projection(logits, lcu, gidx[:R], err)


def lmhead_gather_project(hidden: torch.Tensor, weight: torch.Tensor, cu_seqlens: torch.Tensor,
                          num_decode: int = 0, logits_indices: Optional[torch.Tensor] = None,
                          out_dtype: torch.dtype = torch.float32,
                          logits: Optional[torch.Tensor] = None, variant: int = LMH_HEAD_AUTO,
                          device_error: Optional[torch.Tensor] = None) -> Projection:
    """Gather the sampled rows of a packed batch and project them through the
    head: logits[r] = hidden[src(r)] @ weight.T (weight is [vocab, hidden])."""
    L = lib()
    V, wargs = _dense_weight_args(weight, hidden.shape[1])
    return _project(L.lmhead_gather_project, L.lmh_debug_gather_project, "lmhead_gather_project",
                    hidden, wargs, V, cu_seqlens, num_decode, logits_indices, out_dtype, logits,
                    variant, device_error)


def lmhead_gather_project_q(hidden: torch.Tensor, weight: QuantizedWeight, cu_seqlens: torch.Tensor,
                            num_decode: int = 0, logits_indices: Optional[torch.Tensor] = None,
                            out_dtype: torch.dtype = torch.float32,
                            logits: Optional[torch.Tensor] = None, variant: int = LMH_HEAD_AUTO,
                            device_error: Optional[torch.Tensor] = None) -> Projection:
    """lmhead_gather_project with a quantised head (bf16 hidden states)."""
    L = lib()
    V, wargs = _quant_weight_args(weight, hidden.shape[1])
    return _project(L.lmhead_gather_project_q, L.lmh_debug_gather_project_q,
                    "lmhead_gather_project_q", hidden, wargs, V, cu_seqlens, num_decode,
                    logits_indices, out_dtype, logits, variant, device_error)


class Reduction(NamedTuple):
    lse: torch.Tensor
    selected_logprob: Optional[torch.Tensor]
    topk_ids: torch.Tensor
    topk_logprobs: torch.Tensor
    device_error: torch.Tensor


def logprob_reduce(logits: torch.Tensor, selected_ids: Optional[torch.Tensor] = None, k: int = 0,
                   ws: Optional[torch.Tensor] = None,
                   out: Optional[Reduction] = None) -> Reduction:
    """Per-row logsumexp, selected-token logprob and exact top-K (ties by
    ascending id) of a [rows, vocab] bf16/fp32 logits matrix, on the device."""
    L = lib()
    R, V, ld = _matrix(logits, "logits")
    sel = _i32(selected_ids, "selected_ids")
    dev = logits.device
    need = L.logprob_reduce_workspace_size(R, V, k)
    if ws is None:
        ws = workspace(need, dev)
    if out is None:
        ids, lps = _topk_out(R, V, k, dev)
        out = Reduction(torch.empty(R, dtype=torch.float32, device=dev),
                        torch.empty(R, dtype=torch.float32, device=dev) if sel is not None else None,
                        ids, lps, torch.zeros(1, dtype=torch.int32, device=dev))
    pi, pl = _topk_ptrs(k, out.topk_ids, out.topk_logprobs)
    st = L.logprob_reduce(_ptr(logits), _dt(logits), R, V, ld, _ptr(sel), int(k),
                          _ptr(out.lse), _ptr(out.selected_logprob), pi, pl,
                          _ptr(ws), ws.numel(), _ptr(out.device_error), _stream())
    _check(st, "logprob_reduce")
    return out


def logprob_reduce_noalloc(logits: torch.Tensor, selected_ids: Optional[torch.Tensor] = None,
                           k: int = 0, out: Optional[Reduction] = None) -> Reduction:
    """logprob_reduce on the library's static per-device scratch (no
    workspace argument; the call itself allocates nothing -- pass `out` to
    keep this wrapper from allocating the outputs)."""
    L = lib()
    R, V, ld = _matrix(logits, "logits")
    sel = _i32(selected_ids, "selected_ids")
    dev = logits.device
    if out is None:
        ids, lps = _topk_out(R, V, k, dev)
        out = Reduction(torch.empty(R, dtype=torch.float32, device=dev),
                        torch.empty(R, dtype=torch.float32, device=dev) if sel is not None else None,
                        ids, lps, torch.zeros(1, dtype=torch.int32, device=dev))
    pi, pl = _topk_ptrs(k, out.topk_ids, out.topk_logprobs)
    st = L.logprob_reduce_noalloc(_ptr(logits), _dt(logits), R, V, ld, _ptr(sel), int(k),
                                  _ptr(out.lse), _ptr(out.selected_logprob), pi, pl,
                                  _ptr(out.device_error), _stream())
    _check(st, "logprob_reduce_noalloc")
    return out


def reduce_single(logits: torch.Tensor, selected_ids: Optional[torch.Tensor], k: int,
                  counters: torch.Tensor) -> Reduction:
    """logprob_reduce through the single-launch few-row path at any k it
    supports (lmh_debug_reduce_single); `counters` is an int32 tensor of 4096
    zeros that every call leaves zero."""
    L = lib()
    R, V, ld = _matrix(logits, "logits")
    sel = _i32(selected_ids, "selected_ids")
    dev = logits.device
    ws = workspace(L.logprob_reduce_workspace_size(R, V, k), dev)
    ids, lps = _topk_out(R, V, k, dev)
    out = Reduction(torch.empty(R, dtype=torch.float32, device=dev),
                    torch.empty(R, dtype=torch.float32, device=dev) if sel is not None else None,
                    ids, lps, torch.zeros(1, dtype=torch.int32, device=dev))
    pi, pl = _topk_ptrs(k, out.topk_ids, out.topk_logprobs)
    st = L.lmh_debug_reduce_single(_ptr(logits), _dt(logits), R, V, ld, _ptr(sel), int(k),
                                   _ptr(out.lse), _ptr(out.selected_logprob), pi, pl, _ptr(ws), ws.numel(),
                                   _ptr(counters), _ptr(out.device_error), _stream())
    _check(st, "lmh_debug_reduce_single")
    return out


def reduce_stage1(logits: torch.Tensor, k: int, ws: torch.Tensor) -> None:
    """Only the streaming pass of logprob_reduce (for timing that kernel)."""
    L = lib()
    R, V, ld = _matrix(logits, "logits")
    _check(L.lmh_debug_reduce_stage1(_ptr(logits), _dt(logits), R, V, ld, int(k), _ptr(ws),
                                     ws.numel(), _stream()), "lmh_debug_reduce_stage1")


def reduce_row_path(rows: int, vocab: int, k: int) -> bool:
    """True when logprob_reduce of this shape runs one workgroup per row on
    the current device (a single launch), False for the two-launch path."""
    return bool(lib().lmh_debug_reduce_path(int(rows), int(vocab), int(k)))


class Logprobs(NamedTuple):
    lse: torch.Tensor
    selected_logprob: Optional[torch.Tensor]
    topk_ids: torch.Tensor
    topk_logprobs: torch.Tensor
    logits_cu_seqlens: torch.Tensor
    gather_indices: torch.Tensor
    device_error: torch.Tensor
    logits: Optional[torch.Tensor]


def lmhead_logprobs_workspace_size(rows: int, vocab: int, k: int, chunk_rows: int = 0) -> int:
    return int(lib().lmhead_logprobs_workspace_size(rows, vocab, k, chunk_rows))


def _logprobs(fn, name, hidden, weight_args, V, cu_seqlens, num_decode, selected_ids, k,
              logits_indices, chunk_rows, return_logits, ws) -> Logprobs:
    L = lib()
    T, H, hld = _matrix(hidden, "hidden")
    cu = _i32(cu_seqlens, "cu_seqlens")
    ex = _i32(logits_indices, "logits_indices")
    sel = _i32(selected_ids, "selected_ids")
    S = cu.shape[0] - 1
    R = ex.shape[0] if ex is not None else S
    dev = hidden.device
    if ws is None:
        ws = workspace(L.lmhead_logprobs_workspace_size(R, V, k, chunk_rows), dev)
    ld = (V + 3) // 4 * 4
    dbg = torch.empty((R, ld), dtype=torch.float32, device=dev) if return_logits else None
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    slp = torch.empty(R, dtype=torch.float32, device=dev) if sel is not None else None
    ids, lps = _topk_out(R, V, k, dev)
    lcu = torch.empty(S + 1, dtype=torch.int32, device=dev)
    gidx = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    st = fn(_ptr(hidden), _dt(hidden), T, H, hld, *weight_args,
            _ptr(cu), S, int(num_decode), _ptr(ex), R if ex is not None else 0,
            _ptr(sel), int(k), _ptr(lse), _ptr(slp), *_topk_ptrs(k, ids, lps),
            _ptr(lcu), _ptr(gidx), int(chunk_rows), _ptr(dbg),
            _ptr(ws), ws.numel(), _ptr(err), _stream())
    _check(st, name)
    return Logprobs(lse, slp, ids, lps, lcu, gidx[:R], err,
                    None if dbg is None else dbg[:, :V])


def lmhead_logprobs(hidden: torch.Tensor, weight: torch.Tensor, cu_seqlens: torch.Tensor,
                    num_decode: int = 0, selected_ids: Optional[torch.Tensor] = None, k: int = 0,
                    logits_indices: Optional[torch.Tensor] = None, chunk_rows: int = 0,
                    return_logits: bool = False, ws: Optional[torch.Tensor] = None) -> Logprobs:
    """Fused gather + projection + reduction, chunked (default 256 rows)."""
    V, wargs = _dense_weight_args(weight, hidden.shape[1])
    return _logprobs(lib().lmhead_logprobs, "lmhead_logprobs", hidden, wargs, V, cu_seqlens,
                     num_decode, selected_ids, k, logits_indices, chunk_rows, return_logits, ws)


def lmhead_logprobs_q(hidden: torch.Tensor, weight: QuantizedWeight, cu_seqlens: torch.Tensor,
                      num_decode: int = 0, selected_ids: Optional[torch.Tensor] = None, k: int = 0,
                      logits_indices: Optional[torch.Tensor] = None, chunk_rows: int = 0,
                      return_logits: bool = False, ws: Optional[torch.Tensor] = None) -> Logprobs:
    """lmhead_logprobs with a quantised head (bf16 hidden states)."""
    V, wargs = _quant_weight_args(weight, hidden.shape[1])
    return _logprobs(lib().lmhead_logprobs_q, "lmhead_logprobs_q", hidden, wargs, V, cu_seqlens,
                     num_decode, selected_ids, k, logits_indices, chunk_rows, return_logits, ws)


class HeadSpec(NamedTuple):
    """A head for the *_ex entry points: dense weights ([vocab, hidden]
    tensor) or a QuantizedWeight, and output scaling (LMH_SCALE_MUL multiplies
    the fp32 logits by `scale`, LMH_SCALE_DIV divides them by it)."""
    weight: object
    scale_mode: int = LMH_SCALE_NONE
    scale: float = 1.0


def _head_struct(head: HeadSpec, H: int):
    h = LmhHead()
    if isinstance(head.weight, QuantizedWeight):
        V, a = _quant_weight_args(head.weight, H)
        h.weight, h.weight_dt, h.weight_ld = None, LMH_BF16, 0
        h.weight_q, h.weight_q_ld, h.scales, h.biases, h.scales_ld = a[0], a[1], a[2], a[3], a[4]
        h.bits, h.group_size = a[5], a[6]
    else:
        V, a = _dense_weight_args(head.weight, H)
        h.weight, h.weight_dt, h.weight_ld = a[0], a[1], a[3]
        h.bits, h.group_size = 0, 0
    h.scale_mode, h.scale = int(head.scale_mode), float(head.scale)
    return V, h


def lmhead_gather_project_ex(hidden: torch.Tensor, head: HeadSpec, cu_seqlens: torch.Tensor,
                             num_decode: int = 0, logits_indices: Optional[torch.Tensor] = None,
                             out_dtype: torch.dtype = torch.float32,
                             logits: Optional[torch.Tensor] = None, variant: int = LMH_HEAD_AUTO,
                             device_error: Optional[torch.Tensor] = None) -> Projection:
    """lmhead_gather_project with a HeadSpec (weights and output scaling)."""
    L = lib()
    V, h = _head_struct(head, hidden.shape[1])
    T, H, hld = _matrix(hidden, "hidden")
    cu = _i32(cu_seqlens, "cu_seqlens")
    ex = _i32(logits_indices, "logits_indices")
    S = cu.shape[0] - 1
    R = ex.shape[0] if ex is not None else S
    dev = hidden.device
    if logits is None:
        logits = torch.empty((R, V), dtype=out_dtype, device=dev)
    _, _, old = _matrix(logits, "logits") if R > 0 else (0, 0, V)
    lcu = torch.empty(S + 1, dtype=torch.int32, device=dev)
    gidx = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
    err = device_error if device_error is not None else torch.zeros(1, dtype=torch.int32, device=dev)
    st = L.lmhead_gather_project_ex(_ptr(hidden), _dt(hidden), T, H, hld, ctypes.byref(h), V,
                                    _ptr(cu), S, int(num_decode), _ptr(ex), R if ex is not None else 0,
                                    _ptr(logits), _dt(logits), old, _ptr(lcu), _ptr(gidx), _ptr(err),
                                    _stream(), int(variant))
    _check(st, "lmhead_gather_project_ex")
    return Projection(logits, lcu, gidx[:R], err)


def lmhead_logprobs_ex(hidden: torch.Tensor, head: HeadSpec, cu_seqlens: torch.Tensor,
                       num_decode: int = 0, selected_ids: Optional[torch.Tensor] = None, k: int = 0,
                       logits_indices: Optional[torch.Tensor] = None, chunk_rows: int = 0,
                       return_logits: bool = False, ws: Optional[torch.Tensor] = None,
                       vocab_mask: Optional[torch.Tensor] = None, epilogue: Optional[int] = None) -> Logprobs:
    """lmhead_logprobs with a HeadSpec (the reduction sees the scaled logits)
    and an optional token bitmask ([segments, words] int32, bit v % 32 of
    word v // 32 set = token v kept in that segment's rows), applied to each
    chunk's logits before it is reduced. `epilogue` (diagnostic): None as
    the library chooses; 0 lets the tiled head's epilogue take the
    reduction's first pass where it can, 1 never (lmh_debug_logprobs_ex)."""
    L = lib()
    V, h = _head_struct(head, hidden.shape[1])
    T, H, hld = _matrix(hidden, "hidden")
    cu = _i32(cu_seqlens, "cu_seqlens")
    ex = _i32(logits_indices, "logits_indices")
    sel = _i32(selected_ids, "selected_ids")
    S = cu.shape[0] - 1
    R = ex.shape[0] if ex is not None else S
    dev = hidden.device
    if ws is None:
        ws = workspace(L.lmhead_logprobs_workspace_size(R, V, k, chunk_rows), dev)
    ld = (V + 3) // 4 * 4
    dbg = torch.empty((R, ld), dtype=torch.float32, device=dev) if return_logits else None
    lse = torch.empty(R, dtype=torch.float32, device=dev)
    slp = torch.empty(R, dtype=torch.float32, device=dev) if sel is not None else None
    ids, lps = _topk_out(R, V, k, dev)
    lcu = torch.empty(S + 1, dtype=torch.int32, device=dev)
    gidx = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    mld = 0
    if vocab_mask is not None:
        Sm, _, mld = _matrix(vocab_mask, "vocab_mask")
        if vocab_mask.dtype != torch.int32 or Sm != S:
            raise ValueError("vocab_mask must be int32 words, one row per segment")
    args = (_ptr(hidden), _dt(hidden), T, H, hld, ctypes.byref(h), V,
            _ptr(cu), S, int(num_decode), _ptr(ex), R if ex is not None else 0,
            _ptr(sel), int(k), _ptr(lse), _ptr(slp), *_topk_ptrs(k, ids, lps),
            _ptr(lcu), _ptr(gidx), int(chunk_rows), _ptr(dbg), _ptr(vocab_mask), mld,
            _ptr(ws), ws.numel(), _ptr(err), _stream())
    if epilogue is None:
        _check(L.lmhead_logprobs_ex(*args), "lmhead_logprobs_ex")
    else:
        _check(L.lmh_debug_logprobs_ex(*args, int(epilogue)), "lmh_debug_logprobs_ex")
    return Logprobs(lse, slp, ids, lps, lcu, gidx[:R], err, None if dbg is None else dbg[:, :V])


class SelfCheck(NamedTuple):
    result: torch.Tensor          # int64[2]: differing logits, first r * vocab + v (INT64_MAX: none)
    device_error: torch.Tensor


def lmhead_apply_bitmask(logits: torch.Tensor, bitmask: torch.Tensor,
                         logits_cu_seqlens: Optional[torch.Tensor] = None,
                         device_error: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Token bitmask on compacted logits, in place: segment s (bitmask row s,
    int32 words, bit v % 32 of word v // 32 set = token v kept) covers the
    logits rows logits_cu_seqlens[s] .. [s+1]-1 (None: row s); masked tokens
    become -inf. Returns the device error word."""
    L = lib()
    R, V, ld = _matrix(logits, "logits")
    S, words, mld = _matrix(bitmask, "bitmask")
    if bitmask.dtype != torch.int32:
        raise ValueError("bitmask must be int32 words")
    lcu = _i32(logits_cu_seqlens, "logits_cu_seqlens")
    if lcu is not None and lcu.shape[0] != S + 1:
        raise ValueError("logits_cu_seqlens needs one entry more than bitmask has rows")
    err = device_error if device_error is not None else torch.zeros(1, dtype=torch.int32,
                                                                    device=logits.device)
    _check(L.lmhead_apply_bitmask(_ptr(logits), _dt(logits), R, V, ld, _ptr(bitmask), mld, _ptr(lcu), S,
                                  _ptr(err), _stream()), "lmhead_apply_bitmask")
    return err


def lmhead_selfcheck(hidden: torch.Tensor, head: HeadSpec, cu_seqlens: torch.Tensor,
                     full_logits: torch.Tensor, num_decode: int = 0,
                     logits_indices: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> SelfCheck:
    """Project the selected rows through `head` and compare them bit for bit
    with the rows of `full_logits` ([num_tokens, vocab] fp32, the head's own
    output at every position) they come from."""
    L = lib()
    V, h = _head_struct(head, hidden.shape[1])
    T, H, hld = _matrix(hidden, "hidden")
    Tf, Vf, fld = _matrix(full_logits, "full_logits")
    if full_logits.dtype != torch.float32 or Vf != V or Tf != T:
        raise ValueError("full_logits must be fp32 [num_tokens, vocab]")
    cu = _i32(cu_seqlens, "cu_seqlens")
    ex = _i32(logits_indices, "logits_indices")
    S = cu.shape[0] - 1
    R = ex.shape[0] if ex is not None else S
    dev = hidden.device
    if ws is None:
        ws = workspace(L.lmhead_selfcheck_workspace_size(R, V), dev)
    res = torch.empty(2, dtype=torch.int64, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    st = L.lmhead_selfcheck(_ptr(hidden), _dt(hidden), T, H, hld, ctypes.byref(h), V,
                            _ptr(cu), S, int(num_decode), _ptr(ex), R if ex is not None else 0,
                            _ptr(full_logits), fld, _ptr(ws), ws.numel(), _ptr(res), _ptr(err),
                            _stream())
    _check(st, "lmhead_selfcheck")
    return SelfCheck(res, err)
