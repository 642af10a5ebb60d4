"""Second, independent oracle for small inputs, built from library routines.

TEST INFRASTRUCTURE ONLY (see the package docstring). Each function states
the same quantity as the C oracle through a different route, so that the two
can pin one another:

* rows: a numpy cumulative formula over segment boundaries
  (vllm-metal release v0.4.0, Summary);
* head: ``numpy`` float64 matmul (mlxcel PR #1969: the head acts per
  position);
* lse: ``scipy.special.logsumexp`` (MTPLX PR #532, Change);
* top-K: ``numpy.lexsort`` on (id, -value) -- value descending, exact ties
  by ascending id (MTPLX PR #532, Change).
"""
from __future__ import annotations

import numpy as np
from scipy.special import logsumexp


def widen(a: np.ndarray) -> np.ndarray:
    """float32 / raw-bf16 uint16 / float64 -> float64, exactly."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rows(cu_seqlens, logits_indices=None):
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    S = cu.shape[0] - 1
    if logits_indices is None:
        return (cu[1:] - 1).astype(np.int32), np.arange(S + 1, dtype=np.int32)
    idx = np.asarray(logits_indices, dtype=np.int64)
    lcu = np.searchsorted(np.sort(idx), cu, side="left")
    return idx.astype(np.int32), lcu.astype(np.int32)


def head(hidden, weight, idx):
    h = widen(np.asarray(hidden))[np.asarray(idx)]
    return h @ widen(np.asarray(weight)).T


def reduce(logits, selected=None, k: int = 0):
    x = widen(np.asarray(logits))
    R, V = x.shape
    with np.errstate(invalid="ignore"):
        lse = logsumexp(x, axis=1)
        lp = x - lse[:, None]
    sel_lp = None if selected is None else lp[np.arange(R), np.asarray(selected)]
    ids = np.empty((R, k), dtype=np.int32)
    vals = np.empty((R, k), dtype=np.float64)
    for r in range(R):
        order = np.lexsort((np.arange(V), -x[r]))[:k]
        ids[r] = order
        vals[r] = lp[r, order]
    return lse, sel_lp, ids, vals
