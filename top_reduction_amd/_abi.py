"""ctypes prototypes of liblmhead's C ABI (include/lmhead.h): the library
path, the constants, the lmh_head mirror and the loader. Imports nothing but
the standard library, so the ABI can be loaded and checked without torch."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblmhead.so")

LMH_F32, LMH_BF16, LMH_F16 = 0, 1, 2
LMH_HEAD_AUTO, LMH_HEAD_STREAM, LMH_HEAD_TILED, LMH_HEAD_PIPE = 0, 1, 2, 3
LMH_SCALE_NONE, LMH_SCALE_MUL, LMH_SCALE_DIV = 0, 1, 2
LMH_DEVERR_INDEX, LMH_DEVERR_LAYOUT = 1, 2
LMH_K_FULL = -1   # k: every token's logprob ([rows, vocab] in topk_logprobs) instead of a top-K
STATUS = {0: "LMH_OK", 1: "LMH_ERR_NULL", 2: "LMH_ERR_SHAPE", 3: "LMH_ERR_K",
          4: "LMH_ERR_DTYPE", 5: "LMH_ERR_ALIGN", 6: "LMH_ERR_WORKSPACE", 7: "LMH_ERR_HIP"}


class LmhHead(ctypes.Structure):
    """ctypes mirror of the C `lmh_head` descriptor (include/lmhead.h)."""
    _fields_ = [("weight", ctypes.c_void_p), ("weight_dt", ctypes.c_int), ("weight_ld", ctypes.c_int64),
                ("bits", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("weight_q", ctypes.c_void_p), ("weight_q_ld", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p), ("scales_ld", ctypes.c_int64),
                ("scale_mode", ctypes.c_int32), ("scale", ctypes.c_float)]


class LmhError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library at `path` with every entry point's prototype (raises
    if it has not been built)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    proj = [p, ctypes.c_int, i64, i64, i64, p, ctypes.c_int, i64, i64, p, i32, i32, p, i32]
    L.lmhead_gather_project.argtypes = proj + [p, ctypes.c_int, i64, p, p, p, p]
    L.lmh_debug_gather_project.argtypes = proj + [p, ctypes.c_int, i64, p, p, p, p, i32]
    L.logprob_reduce_workspace_size.argtypes = [i64, i64, i32]
    L.logprob_reduce_workspace_size.restype = sz
    L.logprob_reduce.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i32, p, p, p, p, p, sz, p, p]
    L.logprob_reduce_noalloc.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i32, p, p, p, p, p, p]
    L.lmh_debug_reduce_single.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i32, p, p, p, p, p, sz, p, p, p]
    L.lmh_debug_reduce_stage1.argtypes = [p, ctypes.c_int, i64, i64, i64, i32, p, sz, p]
    L.lmh_debug_reduce_path.argtypes = [i64, i64, i32]
    L.lmh_debug_reduce_path.restype = i32
    L.lmhead_logprobs_workspace_size.argtypes = [i64, i64, i32, i32]
    L.lmhead_logprobs_workspace_size.restype = sz
    L.lmhead_logprobs.argtypes = proj + [p, i32, p, p, p, p, p, p, i32, p, p, sz, p, p]
    projq = [p, ctypes.c_int, i64, i64, i64, p, i64, p, p, i64, i32, i32, i64, p, i32, i32, p, i32]
    L.lmhead_gather_project_q.argtypes = projq + [p, ctypes.c_int, i64, p, p, p, p]
    L.lmh_debug_gather_project_q.argtypes = projq + [p, ctypes.c_int, i64, p, p, p, p, i32]
    L.lmhead_logprobs_q.argtypes = projq + [p, i32, p, p, p, p, p, p, i32, p, p, sz, p, p]
    hp = ctypes.POINTER(LmhHead)
    projx = [p, ctypes.c_int, i64, i64, i64, hp, i64, p, i32, i32, p, i32]
    L.lmhead_gather_project_ex.argtypes = projx + [p, ctypes.c_int, i64, p, p, p, p, i32]
    L.lmhead_logprobs_ex.argtypes = projx + [p, i32, p, p, p, p, p, p, i32, p, p, i64, p, sz, p, p]
    L.lmh_debug_logprobs_ex.argtypes = projx + [p, i32, p, p, p, p, p, p, i32, p, p, i64, p, sz, p, p, i32]
    L.lmhead_selfcheck_workspace_size.argtypes = [i64, i64]
    L.lmhead_selfcheck_workspace_size.restype = sz
    L.lmhead_selfcheck.argtypes = projx + [p, i64, p, sz, p, p, p]
    L.lmhead_apply_bitmask.argtypes = [p, ctypes.c_int, i64, i64, i64, p, i64, p, i32, p, p]
    L.lmh_status_string.argtypes = [ctypes.c_int]
    L.lmh_status_string.restype = ctypes.c_char_p
    for name in ("lmhead_gather_project", "lmh_debug_gather_project", "logprob_reduce",
                 "logprob_reduce_noalloc", "lmh_debug_reduce_single",
                 "lmh_debug_reduce_stage1", "lmhead_logprobs", "lmhead_gather_project_q",
                 "lmh_debug_gather_project_q", "lmhead_logprobs_q", "lmhead_gather_project_ex",
                 "lmhead_logprobs_ex", "lmh_debug_logprobs_ex", "lmhead_selfcheck", "lmhead_apply_bitmask"):
        getattr(L, name).restype = ctypes.c_int
    return L
