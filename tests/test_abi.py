"""The C ABI on the CPU: the library loads without a GPU, exports every entry
point the header declares, and rejects bad host-visible arguments with the
documented status before any HIP call (so no GPU is touched)."""
import ctypes
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead.h")
# the library under test: the build's, or another build of the same sources
# (the sanitizer test runs this module against a host-instrumented build)
LIB = os.environ.get("LMH_TEST_LIBRARY", os.path.join(ROOT, "top_reduction_amd", "liblmhead.so"))


def _abi_module():
    """top_reduction_amd/_abi.py loaded by path: the prototypes without torch."""
    spec = importlib.util.spec_from_file_location("lmh_abi", os.path.join(ROOT, "top_reduction_amd", "_abi.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


ABI = _abi_module()

OK, NULL, SHAPE, K, DTYPE, ALIGN, WS, HIP = range(8)
F32, BF16, F16, BAD_DT = 0, 1, 2, 7
A = 0x10000  # a 256-aligned stand-in address; never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^(?:lmh_status|size_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.skip("liblmhead.so is not built")
    return ABI.load(LIB)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"lmhead_gather_project", "logprob_reduce", "lmhead_logprobs",
            "logprob_reduce_workspace_size", "lmhead_logprobs_workspace_size",
            "lmh_status_string", "lmhead_gather_project_q", "lmhead_logprobs_q"} <= names


def test_every_declared_symbol_is_exported(L):
    raw = ctypes.CDLL(LIB)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_status_strings(L):
    for st in range(8):
        assert L.lmh_status_string(st).decode().startswith("LMH_")


def _project(L, **kw):
    a = dict(hidden=A, hidden_dt=BF16, num_tokens=23, hidden_dim=64, hidden_ld=64, weight=A,
             weight_dt=BF16, vocab=1000, weight_ld=64, cu=A, S=5, D=2, ex=None, nex=0,
             logits=A, logits_dt=F32, logits_ld=1000, lcu=None, gidx=None, err=None)
    a.update(kw)
    return L.lmhead_gather_project(a["hidden"], a["hidden_dt"], a["num_tokens"], a["hidden_dim"],
                                   a["hidden_ld"], a["weight"], a["weight_dt"], a["vocab"],
                                   a["weight_ld"], a["cu"], a["S"], a["D"], a["ex"], a["nex"],
                                   a["logits"], a["logits_dt"], a["logits_ld"], a["lcu"], a["gidx"],
                                   a["err"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(hidden=None), NULL), (dict(weight=None), NULL), (dict(cu=None), NULL),
    (dict(logits=None), NULL),
    (dict(num_tokens=0), SHAPE), (dict(hidden_dim=0), SHAPE), (dict(vocab=0), SHAPE),
    (dict(S=-1), SHAPE), (dict(D=6), SHAPE), (dict(D=-1), SHAPE),
    (dict(hidden_ld=32), SHAPE), (dict(weight_ld=63), SHAPE), (dict(logits_ld=999), SHAPE),
    (dict(ex=A, nex=-1), SHAPE),
    (dict(hidden_dt=BAD_DT, weight_dt=BAD_DT), DTYPE), (dict(weight_dt=F32), DTYPE),
    (dict(hidden_dt=F16, weight_dt=F16), DTYPE), (dict(logits_dt=F16), DTYPE),   # f16: reduction only
    (dict(logits_dt=BAD_DT), DTYPE),
    (dict(hidden=A + 8), ALIGN), (dict(weight=A + 2), ALIGN), (dict(hidden_dim=60, hidden_ld=64), ALIGN),
    (dict(hidden_ld=68), ALIGN), (dict(logits=A + 2), ALIGN),
])
def test_gather_project_rejects(L, kw, want):
    assert _project(L, **kw) == want


def test_debug_variant_rules(L):
    args = [A, BF16, 200, 64, 64, A, BF16, 1000, 64, A, 100, 0, None, 0, A, F32, 1000, None, None, None, None]
    assert L.lmh_debug_gather_project(*args, 1) == SHAPE      # streaming head needs R <= 64
    assert L.lmh_debug_gather_project(*args, 3) == SHAPE      # unknown variant
    f32 = list(args)
    f32[1] = f32[6] = F32
    f32[9] = A
    f32[10] = 5
    assert L.lmh_debug_gather_project(*f32, 2) == SHAPE       # variants are bf16-only


def _project_q(L, debug_variant=None, **kw):
    a = dict(hidden=A, hidden_dt=BF16, num_tokens=23, hidden_dim=128, hidden_ld=128, q=A, q_ld=16,
             scales=A, biases=A, s_ld=2, bits=4, group=64, vocab=1000, cu=A, S=5, D=2, ex=None,
             nex=0, logits=A, logits_dt=F32, logits_ld=1000, lcu=None, gidx=None, err=None)
    a.update(kw)
    args = [a["hidden"], a["hidden_dt"], a["num_tokens"], a["hidden_dim"], a["hidden_ld"], a["q"],
            a["q_ld"], a["scales"], a["biases"], a["s_ld"], a["bits"], a["group"], a["vocab"],
            a["cu"], a["S"], a["D"], a["ex"], a["nex"], a["logits"], a["logits_dt"],
            a["logits_ld"], a["lcu"], a["gidx"], a["err"], None]
    if debug_variant is None:
        return L.lmhead_gather_project_q(*args)
    return L.lmh_debug_gather_project_q(*args, debug_variant)


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), NULL), (dict(scales=None), NULL), (dict(biases=None), NULL),
    (dict(bits=3), DTYPE), (dict(bits=16), DTYPE), (dict(hidden_dt=F32), DTYPE),
    (dict(group=16), SHAPE), (dict(group=256), SHAPE), (dict(group=48), SHAPE),
    (dict(hidden_dim=64, hidden_ld=64, q_ld=8, s_ld=1), SHAPE),
    (dict(q_ld=12), SHAPE), (dict(bits=8, q_ld=16), SHAPE), (dict(s_ld=1), SHAPE),
    (dict(group=32, s_ld=3), SHAPE),
    (dict(q_ld=18), ALIGN), (dict(q=A + 8), ALIGN), (dict(scales=A + 1), ALIGN),
    (dict(biases=A + 3), ALIGN), (dict(hidden=A + 8), ALIGN),
    (dict(num_tokens=0), SHAPE), (dict(vocab=0), SHAPE), (dict(logits_ld=999), SHAPE),
])
def test_gather_project_q_rejects(L, kw, want):
    assert _project_q(L, **kw) == want


def test_debug_variant_rules_q(L):
    assert _project_q(L, debug_variant=1, S=100, D=0) == SHAPE   # streaming head needs R <= 64
    assert _project_q(L, debug_variant=3) == SHAPE               # unknown variant


def _reduce(L, **kw):
    a = dict(logits=A, dt=BF16, rows=256, vocab=248320, ld=248320, sel=A, k=20, lse=A, slp=A,
             ids=A, lps=A, ws=A, wsb=1 << 30, err=None)
    a.update(kw)
    return L.logprob_reduce(a["logits"], a["dt"], a["rows"], a["vocab"], a["ld"], a["sel"], a["k"],
                            a["lse"], a["slp"], a["ids"], a["lps"], a["ws"], a["wsb"], a["err"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(logits=None), NULL), (dict(lse=None), NULL), (dict(slp=None), NULL),
    (dict(ids=None), NULL), (dict(lps=None), NULL),
    (dict(rows=-1), SHAPE), (dict(vocab=0), SHAPE), (dict(ld=248319), SHAPE),
    (dict(dt=BAD_DT), DTYPE),
    (dict(logits=A + 8), ALIGN), (dict(ld=248324), ALIGN),
    (dict(dt=F16, wsb=1024), WS), (dict(dt=F16, ld=248324), ALIGN),   # f16 logits are accepted
    (dict(k=-2), K), (dict(k=129), K), (dict(vocab=100, ld=104, k=101), K),
    (dict(k=-1, lps=None), NULL), (dict(k=-1, ids=None, wsb=16), WS),   # full-vocabulary mode
    (dict(vocab=9 * 8192 * 64, ld=9 * 8192 * 64, k=1), SHAPE),
    (dict(ws=None), WS), (dict(wsb=1024), WS), (dict(ws=A + 16), WS),
])
def test_reduce_rejects(L, kw, want):
    assert _reduce(L, **kw) == want


def test_reduce_k_rule_small_vocab(L):
    # V <= 8192: any K <= V passes the K rule (so the workspace check is reached)
    assert _reduce(L, vocab=8192, ld=8192, k=8192, wsb=16) == WS
    assert _reduce(L, vocab=8256, ld=8256, k=129, wsb=16) == K


def test_reduce_zero_rows_is_a_noop(L):
    assert _reduce(L, rows=0, logits=None, lse=None, slp=None, ids=None, lps=None, ws=None) == OK
    assert _reduce(L, rows=0, k=129) == K


def test_reduce_k0_needs_no_topk_buffers(L):
    assert _reduce(L, k=0, ids=None, lps=None, wsb=16) == WS


def _reduce_noalloc(L, **kw):
    a = dict(logits=A, dt=BF16, rows=256, vocab=248320, ld=248320, sel=A, k=20, lse=A, slp=A,
             ids=A, lps=A, err=None)
    a.update(kw)
    return L.logprob_reduce_noalloc(a["logits"], a["dt"], a["rows"], a["vocab"], a["ld"], a["sel"], a["k"],
                                    a["lse"], a["slp"], a["ids"], a["lps"], a["err"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(logits=None), NULL), (dict(lse=None), NULL), (dict(slp=None), NULL),
    (dict(ids=None), NULL), (dict(lps=None), NULL),
    (dict(rows=-1), SHAPE), (dict(vocab=0), SHAPE), (dict(ld=248319), SHAPE),
    (dict(dt=BAD_DT), DTYPE), (dict(logits=A + 8), ALIGN),
    (dict(k=-2), K), (dict(k=129), K), (dict(k=-1, lps=None), NULL),
    # a shape whose reduction workspace is above the static scratch
    (dict(rows=3000), WS), (dict(rows=600, k=0), WS),
])
def test_reduce_noalloc_rejects(L, kw, want):
    """The no-allocation reduction applies logprob_reduce's rules and refuses
    shapes whose scratch exceeds LMH_NOALLOC_SCRATCH_BYTES, all before any
    HIP call."""
    assert _reduce_noalloc(L, **kw) == want


def test_reduce_noalloc_limit(L):
    limit = 8 << 20
    text = open(HEADER).read()
    assert re.search(r"#define LMH_NOALLOC_SCRATCH_BYTES \(\(size_t\)8 << 20\)", text)
    assert L.logprob_reduce_workspace_size(3000, 248320, 20) > limit
    assert L.logprob_reduce_workspace_size(600, 248320, 0) > limit
    assert L.logprob_reduce_workspace_size(32, 151936, 5) <= limit
    assert _reduce_noalloc(L, rows=0, logits=None, lse=None, slp=None, ids=None, lps=None) == OK


def _reduce_single(L, **kw):
    a = dict(logits=A, dt=BF16, rows=32, vocab=151936, ld=151936, sel=A, k=5, lse=A, slp=A,
             ids=A, lps=A, ws=A, wsb=1 << 30, cnt=A, err=None)
    a.update(kw)
    return L.lmh_debug_reduce_single(a["logits"], a["dt"], a["rows"], a["vocab"], a["ld"], a["sel"], a["k"],
                                     a["lse"], a["slp"], a["ids"], a["lps"], a["ws"], a["wsb"], a["cnt"],
                                     a["err"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(logits=None), NULL), (dict(lse=None), NULL), (dict(dt=BAD_DT), DTYPE),
    (dict(logits=A + 8), ALIGN), (dict(k=-2), K), (dict(ws=None), WS), (dict(wsb=16), WS),
    (dict(cnt=None), NULL),
])
def test_reduce_single_rejects(L, kw, want):
    """The forcing entry point of the single-launch path applies
    logprob_reduce's rules, then needs its counters, before any HIP call."""
    assert _reduce_single(L, **kw) == want


def test_workspace_sizes(L):
    for rows, V, k in [(256, 248320, 128), (32, 151936, 5), (1, 1000, 0), (0, 64, 0)]:
        n = L.logprob_reduce_workspace_size(rows, V, k)
        assert n >= 256 and n % 256 == 0
        nb = -(-V // 64)
        assert n >= rows * nb * 2
    a = L.lmhead_logprobs_workspace_size(1024, 128256, 20, 256)
    b = L.lmhead_logprobs_workspace_size(40, 128256, 20, 256)
    assert a >= 256 * 128256 * 4 and b >= 40 * 128256 * 4 and a > b


def test_fused_rejects(L):
    base = [A, BF16, 10272, 4096, 4096, A, BF16, 128256, 4096, A, 40, 32, None, 0,
            A, 20, A, A, A, A, None, None, 0, None, A, 1 << 34, None, None]
    bad = list(base)
    bad[16] = None                      # lse
    assert L.lmhead_logprobs(*bad) == NULL
    bad = list(base)
    bad[15] = 129                       # K rule
    assert L.lmhead_logprobs(*bad) == K
    bad = list(base)
    bad[25] = 1024                      # workspace too small
    assert L.lmhead_logprobs(*bad) == WS
    bad = list(base)
    bad[22] = -1                        # chunk_rows
    assert L.lmhead_logprobs(*bad) == SHAPE


def _head(**kw):
    h = ABI.LmhHead()
    h.weight, h.weight_dt, h.weight_ld, h.bits, h.group_size = A, BF16, 64, 0, 0
    h.weight_q, h.weight_q_ld, h.scales, h.biases, h.scales_ld = None, 0, None, None, 0
    h.scale_mode, h.scale = 0, 1.0
    for k, v in kw.items():
        setattr(h, k, v)
    return h


def _project_ex(L, head, **kw):
    a = dict(hidden=A, hidden_dt=BF16, num_tokens=23, hidden_dim=64, hidden_ld=64, vocab=1000, cu=A,
             S=5, D=2, ex=None, nex=0, logits=A, logits_dt=F32, logits_ld=1000, variant=0)
    a.update(kw)
    return L.lmhead_gather_project_ex(a["hidden"], a["hidden_dt"], a["num_tokens"], a["hidden_dim"],
                                      a["hidden_ld"], None if head is None else ctypes.byref(head),
                                      a["vocab"], a["cu"], a["S"], a["D"], a["ex"], a["nex"],
                                      a["logits"], a["logits_dt"], a["logits_ld"], None, None, None,
                                      None, a["variant"])


@pytest.mark.parametrize("hkw,want", [
    (dict(scale_mode=3), SHAPE), (dict(scale_mode=-1), SHAPE),
    (dict(scale_mode=1, scale=0.0), SHAPE), (dict(scale_mode=2, scale=0.0), SHAPE),
    (dict(scale_mode=1, scale=float("nan")), SHAPE), (dict(scale_mode=2, scale=float("inf")), SHAPE),
    (dict(weight=None), NULL), (dict(weight_dt=F32), DTYPE),
    (dict(bits=4, group_size=64), NULL),                        # quantised without codes
    (dict(weight=A + 2), ALIGN),
])
def test_gather_project_ex_rejects(L, hkw, want):
    assert _project_ex(L, _head(**hkw)) == want


def test_gather_project_ex_null_head_and_variant(L):
    assert _project_ex(L, None) == NULL
    assert _project_ex(L, _head(), variant=3) == SHAPE
    assert _project_ex(L, _head(), S=100, D=0, variant=1) == SHAPE


def test_logprobs_ex_mask_rules(L):
    """The token bitmask of the fused call: a pitch below ceil(vocab/32)
    words, a misaligned mask, and explicit rows without logits_cu_seqlens
    (the segment bounds the mask needs) are refused; a valid mask passes its
    checks (the too-small workspace is what stops the call)."""
    h = _head()

    def call(mask, mask_ld, ex=None, nex=0, lcu=None, wsb=1 << 30):
        return L.lmhead_logprobs_ex(A, BF16, 23, 64, 64, ctypes.byref(h), 1000, A, 5, 2, ex, nex, A, 5,
                                    A, A, A, A, lcu, None, 0, None, mask, mask_ld, A, wsb, None, None)
    assert call(A, 31) == SHAPE
    assert call(A + 2, 32) == ALIGN
    assert call(A, 32, ex=A, nex=5) == NULL
    assert call(A, 32, wsb=16) == WS
    assert call(A, 32, ex=A, nex=5, lcu=A, wsb=16) == WS
    assert call(None, 0, wsb=16) == WS
    assert L.lmhead_logprobs_ex(None, BF16, 23, 64, 64, ctypes.byref(h), 1000, A, 5, 2, None, 0,
                                A, 5, A, A, A, A, None, None, 0, None, None, 0, A, 1 << 30, None,
                                None) == NULL


def test_selfcheck_rejects(L):
    h = _head()
    base = [A, BF16, 23, 64, 64, ctypes.byref(h), 1000, A, 5, 2, None, 0]
    need = L.lmhead_selfcheck_workspace_size(5, 1000)
    assert need == 5 * 1000 * 4 + (256 - 5 * 1000 * 4 % 256) % 256
    assert L.lmhead_selfcheck(*base, None, 1000, A, need, A, None, None) == NULL       # no full logits
    assert L.lmhead_selfcheck(*base, A, 1000, A, need, None, None, None) == NULL       # no result
    assert L.lmhead_selfcheck(*base, A, 999, A, need, A, None, None) == SHAPE          # full_ld < vocab
    assert L.lmhead_selfcheck(*base, A, 1000, A, need - 1, A, None, None) == WS
    assert L.lmhead_selfcheck(*base, A, 1000, None, need, A, None, None) == WS
    assert L.lmhead_selfcheck(*base, A + 2, 1000, A, need, A, None, None) == ALIGN
    assert L.lmhead_selfcheck(*base, A, 1000, A, need, A + 4, None, None) == ALIGN


def test_head_struct_layout_matches_c(tmp_path):
    """The ctypes mirror of lmh_head has C's size and field offsets (compiled
    against include/lmhead.h with the host C compiler)."""
    import subprocess
    fields = [f for f, _ in ABI.LmhHead._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "lmhead.h"\nint main(void){\n'
                   + 'printf("%zu\\n", sizeof(lmh_head));\n'
                   + "".join(f'printf("%zu\\n", offsetof(lmh_head, {f}));\n' for f in fields)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(ABI.LmhHead)
    assert out[1:] == [getattr(ABI.LmhHead, f).offset for f in fields]


def _bitmask(L, **kw):
    a = dict(logits=A, dt=BF16, rows=4, vocab=1000, ld=1000, mask=A, mld=32, lcu=A, S=3, err=None)
    a.update(kw)
    return L.lmhead_apply_bitmask(a["logits"], a["dt"], a["rows"], a["vocab"], a["ld"], a["mask"],
                                  a["mld"], a["lcu"], a["S"], a["err"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(rows=-1), SHAPE), (dict(vocab=0), SHAPE), (dict(ld=999), SHAPE), (dict(mld=31), SHAPE),
    (dict(S=-1), SHAPE), (dict(lcu=None), SHAPE), (dict(dt=BAD_DT), DTYPE),
    (dict(logits=None), NULL), (dict(mask=None), NULL),
    (dict(logits=A + 8), ALIGN), (dict(ld=1004), ALIGN), (dict(mask=A + 2), ALIGN),
])
def test_bitmask_rejects(L, kw, want):
    assert _bitmask(L, **kw) == want


def test_bitmask_no_segments_is_a_no_op(L):
    assert _bitmask(L, logits=None, mask=None, lcu=None, S=0, rows=0) == OK
