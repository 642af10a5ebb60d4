"""CPU oracle for the selective LM head and the per-row logprob reduction.

TEST INFRASTRUCTURE ONLY: imported by the test suite, by the smoke check and
by the benchmark's CPU-baseline leg, never by the product package. It shares
no code with the HIP path; both consume the seeded inputs of ``synth``.

Two independent implementations live here:

* ``liboracle.so`` (``oracle.c``): the plain definition in f64 -- the row
  formula, a naive triple-loop head, a max pass plus an f64 exp-sum pass for
  the logsumexp, a full sort for the top-K (value descending, exact ties
  by ascending token id), the exact dequantisation of affine
  group-quantised head weights, and a token bitmask applied to the
  compacted logits rows of each segment. Thin numpy wrappers below.
* ``ref_numpy``: the same quantities through library routines
  (``numpy`` float64 matmul, ``scipy.special.logsumexp``, ``numpy.lexsort``),
  used to cross-check the C oracle on small inputs.

Parity unpinned: nothing. Every function is pinned by tests against closed
forms, library routines, exhaustive enumeration, integer arithmetic or
hand-worked fixtures (see the oracle tests).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_TEST_LIBRARY: another build of oracle.c to load instead (the
# sanitizer test runs the pins against an instrumented build)
_LIB_PATH = os.environ.get("ORACLE_TEST_LIBRARY", os.path.join(_HERE, "liboracle.so"))
_SRC = os.path.join(_HERE, "oracle.c")

F32, BF16, F64, F16 = 0, 1, 2, 3
OK, ERR_LAYOUT, ERR_INDEX = 0, 1, 2
BLOCK = 64

_lib = None


def build(out: str = _LIB_PATH, extra_flags=()) -> str:
    """Compile oracle.c with gcc (no fast-math) into a shared library."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", *extra_flags, _SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str = _LIB_PATH):
    global _lib
    if _lib is not None and path == _LIB_PATH:
        return _lib
    if not os.path.exists(path):
        build(path)
    lib = ctypes.CDLL(path)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.orc_rows.argtypes = [p, i32, i32, i64, p, i32, p, p]
    lib.orc_rows.restype = ctypes.c_int
    lib.orc_head.argtypes = [p, ctypes.c_int, i64, i64, i64, p, ctypes.c_int, i64, i64, p, i32, p]
    lib.orc_head.restype = None
    lib.orc_dequant.argtypes = [p, i64, p, p, i64, ctypes.c_int, ctypes.c_int, i64, i64, p]
    lib.orc_dequant.restype = None
    lib.orc_scale_logits.argtypes = [p, i64, ctypes.c_int, ctypes.c_double]
    lib.orc_scale_logits.restype = None
    lib.orc_widen.argtypes = [p, ctypes.c_int, i64, p]
    lib.orc_widen.restype = None
    lib.orc_reduce.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i32, p, p, p, p]
    lib.orc_reduce.restype = None
    lib.orc_prefilter_check.argtypes = [p, ctypes.c_int, i64, i64, i64, i32, i32, i32, p]
    lib.orc_prefilter_check.restype = ctypes.c_int64
    lib.orc_apply_bitmask.argtypes = [p, i64, i64, i64, p, i64, p, i32]
    lib.orc_apply_bitmask.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    if path == _LIB_PATH:
        _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:     # raw bf16 bits
        return BF16
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"unsupported oracle dtype {a.dtype}")


def widen(a: np.ndarray, lib=None) -> np.ndarray:
    """The oracle's exact f64 value of every element of a float32, raw-bf16
    (uint16), float16 or float64 array."""
    lib = lib or load()
    a = np.ascontiguousarray(a)
    out = np.empty(a.size, dtype=np.float64)
    lib.orc_widen(_ptr(a), _dtype_code(a), a.size, _ptr(out))
    return out.reshape(a.shape)


def num_threads(lib=None) -> int:
    return (lib or load()).orc_num_threads()


def rows(cu_seqlens, num_decode: int, num_tokens: int, logits_indices=None, lib=None):
    """Row targets. Returns (status, gather_indices[R], logits_cu_seqlens[S+1])."""
    lib = lib or load()
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    S = cu.shape[0] - 1
    if logits_indices is None:
        ex, R = None, S
    else:
        ex = np.ascontiguousarray(logits_indices, dtype=np.int32)
        R = ex.shape[0]
    idx = np.full(R, -1, dtype=np.int32)
    lcu = np.full(S + 1, -1, dtype=np.int32)
    st = lib.orc_rows(_ptr(cu), S, num_decode, num_tokens, _ptr(ex), 0 if ex is None else R,
                      _ptr(idx), _ptr(lcu))
    return st, idx, lcu


SCALE_NONE, SCALE_MUL, SCALE_DIV = 0, 1, 2


def head(hidden: np.ndarray, weight: np.ndarray, idx, lib=None, scale_mode: int = SCALE_NONE,
         scale: float = 1.0) -> np.ndarray:
    """f64 logits Z[r][v] = sum_k hidden[idx[r]][k] * weight[v][k] (k ascending),
    then multiplied by `scale` (SCALE_MUL) or divided by it (SCALE_DIV).
    hidden [T][H] and weight [V][H] are float32 or raw-bf16 uint16 (2-D, any
    row pitch through numpy strides is flattened to a contiguous copy)."""
    lib = lib or load()
    hidden = np.ascontiguousarray(hidden)
    weight = np.ascontiguousarray(weight)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, H = hidden.shape
    V, H2 = weight.shape
    assert H == H2
    Z = np.empty((idx.shape[0], V), dtype=np.float64)
    lib.orc_head(_ptr(hidden), _dtype_code(hidden), T, H, H, _ptr(weight), _dtype_code(weight),
                 V, H, _ptr(idx), idx.shape[0], _ptr(Z))
    lib.orc_scale_logits(_ptr(Z), Z.size, int(scale_mode), float(scale))
    return Z


def dequant(q: np.ndarray, scales: np.ndarray, biases: np.ndarray, bits: int, group: int,
            hidden: int, lib=None) -> np.ndarray:
    """Exact f64 weights [V][hidden] of MLX-style affine group quantisation:
    W[v][k] = scale[v][k // group] * q(v, k) + bias[v][k // group], with q
    unsigned `bits`-bit (4 or 8) integers packed little-endian into the uint32
    words of q [V][words]; scales and biases are raw-bf16 uint16 [V][groups]."""
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.uint32)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    biases = np.ascontiguousarray(biases, dtype=np.uint16)
    V, words = q.shape
    assert words * 32 >= hidden * bits and scales.shape == biases.shape and scales.shape[0] == V
    assert scales.shape[1] * group >= hidden
    W = np.empty((V, hidden), dtype=np.float64)
    lib.orc_dequant(_ptr(q), words, _ptr(scales), _ptr(biases), scales.shape[1], bits, group, V, hidden,
                    _ptr(W))
    return W


def reduce(logits: np.ndarray, selected=None, k: int = 0, lib=None):
    """f64 reduction of each row: (lse[rows], selected_logprob[rows] or None,
    topk_ids[rows][k], topk_logprobs[rows][k])."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    R, V = logits.shape
    lse = np.empty(R, dtype=np.float64)
    sel = None if selected is None else np.ascontiguousarray(selected, dtype=np.int32)
    sel_lp = None if sel is None else np.empty(R, dtype=np.float64)
    ids = np.empty((R, k), dtype=np.int32)
    lp = np.empty((R, k), dtype=np.float64)
    lib.orc_reduce(_ptr(logits), _dtype_code(logits), R, V, V, _ptr(sel), k,
                   _ptr(lse), _ptr(sel_lp), _ptr(ids) if k else None, _ptr(lp) if k else None)
    return lse, sel_lp, ids, lp


def full_logprobs(logits: np.ndarray, lib=None) -> np.ndarray:
    """Every token's logprob, f64 [rows][V]: x - lse of its row (openinfer
    issue #719, Acceptance criteria: -1 asks for the full vocabulary), with
    lse from the plain reduction above; a row of -inf gives NaN (-inf minus
    -inf)."""
    lib = lib or load()
    x = np.ascontiguousarray(widen(logits, lib))
    lse = reduce(logits, None, 0, lib)[0]
    with np.errstate(invalid="ignore"):
        return x - lse[:, None]


def apply_bitmask(logits: np.ndarray, mask: np.ndarray, logits_cu_seqlens=None, lib=None):
    """f64 copy of ``logits`` [rows][V] with segment s's token bitmask (uint32
    words [S][ceil(V/32)], bit set = token kept) applied to its rows
    logits_cu_seqlens[s] .. [s+1]-1 (None: segment s is row s): (status,
    masked f64 logits)."""
    lib = lib or load()
    Z = np.ascontiguousarray(widen(logits, lib))
    R, V = Z.shape
    mask = np.ascontiguousarray(mask, dtype=np.uint32)
    S = mask.shape[0]
    lcu = None if logits_cu_seqlens is None else np.ascontiguousarray(logits_cu_seqlens, dtype=np.int32)
    if lcu is not None:
        assert lcu.shape[0] == S + 1
    else:
        assert S == R
    st = lib.orc_apply_bitmask(_ptr(Z), R, V, V, _ptr(mask), mask.shape[1], _ptr(lcu), S)
    return int(st), Z


def prefilter_check(logits: np.ndarray, k: int, block: int = BLOCK, lib=None,
                    block_ties_descending: bool = False):
    """(failing_rows, candidates_per_row) of the block-max prefilter invariant.
    ``block_ties_descending`` selects a deliberately wrong block tie-break."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    R, V = logits.shape
    cand = np.empty(R, dtype=np.int64)
    fails = lib.orc_prefilter_check(_ptr(logits), _dtype_code(logits), R, V, V, k, block,
                                    int(block_ties_descending), _ptr(cand))
    return int(fails), cand
