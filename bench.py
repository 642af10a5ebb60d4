#!/usr/bin/env python3
"""Benchmark of the selective LM head and the on-device logprob reduction on
one MI355X.

Headline (the JSON line's `value`): logprob-reduce rows/s on the
prompt-scoring chunk -- 256 rows x 248,320 vocabulary bf16 logits, K = 20
(MTPLX PR #532, Motivation and Evidence) -- one `logprob_reduce` call per
step (on a 256-CU device: one launch, a workgroup per row), inputs resident
in HBM, four distinct chunks rotated so that no step is served from the
256 MB MALL.

The same line carries:
  roofline      the step's kernel (streaming pass and top-K in one launch)
                against the 8 TB/s HBM peak, back-to-back launches timed live
                with HIP events; split_stage1 is the streaming kernel of the
                two-launch path (rows that do not fill the CUs) alone;
  cpu_baseline  the f64 CPU oracle on a bounded sample of the same chunk;
  reduce_by_k   the chunk at K = 0, 1, 20, 128;
  decode        32 x 151,936 decode rows, K = 5 (openinfer issue #719);
  head          Qwen3-0.6B-shaped selective head (40 of 81,920 rows) and the
                full 2048-row projection (vllm-metal release, Benchmarks);
  headq         the same head with 4- and 8-bit group-quantised weights
                (mlxcel PR #1969: the measured models are 4-bit);
  fused         Llama-3-8B-shaped fused head + logprobs, mixed batch and a
                1024-token prompt in 256-row chunks.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--sections ...]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
METRIC = "logprob-reduce rows/s & GB/s vs HBM peak; sampled-row LM-head ms"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def ingest_pmc(fetch_csv: str, write_csv: str, out: str = TRAFFIC_FILE) -> None:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, both with --sections copycal,reduce,head,headq,fused) into HBM
    bytes per launch.
    Each counter is scaled by what it reads for the plain elementwise copy of
    known size that the copycal section runs."""
    import csv
    import statistics

    # medians per (kernel, grid size): one kernel name serves several shapes
    def per_kernel(path, counter):
        d = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                d.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return {k: statistics.median(v) for k, v in d.items()}

    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    copy = [k for k in fetch if "vectorized_elementwise_kernel" in k[0]]
    if len(copy) != 1:
        raise SystemExit(f"expected one elementwise copy kernel, found {copy}")
    nbytes = 256 * 248320 * 2
    f_fetch = fetch[copy[0]] * 1024 / nbytes
    f_write = write[copy[0]] * 1024 / nbytes
    csrc = os.path.join(ROOT, "top_reduction_amd", "csrc")
    # (kernel name part, source, algorithmic bytes per launch, grid size in
    # threads or None for any)
    llama_w = 128256 * 4096 * 2
    wanted = {"reduce_row_bf16": ("k_rowreduce<1, 16, true>", "reduce.hip", nbytes, None),
              "reduce_stage1_bf16": ("k_stage1<1, true>", "reduce.hip", nbytes, None),
              "reduce_stage2_bf16": ("k_stage2<1", "reduce.hip", None, None),
              # the Llama-3-8B mixed batch's 40 sampled rows (hidden 4096)
              "head_stream_bf16": ("k_head_stream<", "head.hip", llama_w + 40 * 4096 * 2 + 40 * 128256 * 4, None),
              "head_pipe_bf16": ("k_head_pipe<3, 2, 4, false, false, true>", "pipe.hip",
                                 151936 * 1024 * 2 + 40 * 1024 * 2 + 40 * 151936 * 4, None),
              # the Qwen3-0.6B 2048-row projection (4752 tiles walked by one
              # workgroup of 512 per CU)
              "head_tiled_bf16": ("k_head_tiled64<false, false, true, 16>", "head.hip",
                                  151936 * 1024 * 2 + 2048 * 1024 * 2 + 2048 * 151936 * 4, None),
              # a Llama-3-8B prompt chunk of 256 rows, without and with the
              # reduction's first pass in the epilogue (then per block an
              # 8-byte partial and a 4-byte key as well)
              "head_tiled_chunk_bf16": ("k_head_tiled64<false, false, false, 16>", "head.hip",
                                        llama_w + 256 * 4096 * 2 + 256 * 128256 * 4, 504 * 512),
              "head_tiled_epilogue_bf16": ("k_head_tiled64<false, true, false, 16>", "head.hip",
                                           llama_w + 256 * 4096 * 2 + 256 * 128256 * 4 + 256 * 2004 * 12,
                                           504 * 512),
              "reduce_stage2_blocks": ("k_stage2<0, 8, true>", "reduce.hip", None, None)}
    for bits in (4, 8):
        qbytes = 151936 * 1024 * bits // 8 + 151936 * 16 * 4
        wanted[f"head_stream_q{bits}"] = (f"k_head_stream_q<3, 1, {bits}, ", "head.hip",
                                          qbytes + 40 * 1024 * 2 + 40 * 151936 * 4, None)
        # 4-bit: the 64-wide-stage kernel; 8-bit: the 32-wide one
        pat = "k_head_tiled64<false, false, false, 4>" if bits == 4 else f"k_head_tiled<false, {bits}, "
        wanted[f"head_tiled_q{bits}"] = (pat, "head.hip", qbytes + 2048 * 1024 * 2 + 2048 * 151936 * 4, None)
    res = {"calibration": {"kernel": copy[0][0][:80], "bytes_read": nbytes, "bytes_written": nbytes,
                           "fetch_kib": fetch[copy[0]], "write_kib": write[copy[0]],
                           "fetch_factor": round(f_fetch, 5), "write_factor": round(f_write, 5)}}
    for key, (pat, src, algo, grid) in wanted.items():
        names = [k for k in fetch if pat in k[0] and (grid is None or k[1] == grid)]
        if not names:
            continue
        k = names[0]
        t = fetch[k] * 1024 / f_fetch + write.get(k, 0.0) * 1024 / f_write
        res[key] = {"kernel": k[0][:80], "grid_threads": k[1], "fetch_kib_per_dispatch": fetch[k],
                    "write_kib_per_dispatch": write.get(k), "bytes_per_launch": round(t),
                    "algorithmic_bytes": algo,
                    "source_sha256": source_sha(os.path.join(csrc, src))}
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sections", default="reduce,decode,head,headq,fused,cpu")
    ap.add_argument("--k", type=int, default=20)
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc runs and exit")
    return ap.parse_args()


def source_sha(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def load_traffic(kernel: str, src: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    the kernel's source has changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            entries = json.load(f)
    except (OSError, ValueError):
        return None
    e = entries.get(kernel)
    if not e or e.get("source_sha256") != source_sha(src):
        return None
    return e.get("bytes_per_launch")


class Timer:
    """HIP-event timing on torch's current stream (the stream every call here
    is enqueued on). Before each timed region a spin kernel keeps the GPU busy
    while the launches queue up, so host-side launch cost does not leak into
    the measured intervals."""

    def __init__(self, torch):
        self.torch = torch

    def prime(self, ms=30.0):
        try:
            self.torch.cuda._sleep(int(ms * 1e-3 * 2.1e9))
        except (AttributeError, RuntimeError):
            pass

    def loop_median(self, fns, steps, warmup, reps=5):
        """Median over `reps` short back-to-back loops (limits the drift of a
        long sustained run) of the ms per call."""
        n = max(steps // reps, 10)
        return float(np.median([self.loop(fns, n, warmup if r == 0 else 2) for r in range(reps)]))

    def loop(self, fns, steps, warmup):
        """ms per call of a back-to-back loop over `fns` (rotating)."""
        torch = self.torch
        for i in range(warmup):
            fns[i % len(fns)]()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        self.prime()
        a.record()
        for i in range(steps):
            fns[i % len(fns)]()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def each(self, fns, steps, warmup):
        """Per-launch durations (ms): an event pair around every call."""
        torch = self.torch
        for i in range(warmup):
            fns[i % len(fns)]()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        self.prime()
        for i in range(steps):
            ev[i][0].record()
            fns[i % len(fns)]()
            ev[i][1].record()
        torch.cuda.synchronize()
        return np.array([x.elapsed_time(y) for x, y in ev])


def vp(t):
    return ctypes.c_void_p(t.data_ptr())


def main():
    args = parse()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        if int(os.environ.get("RANK", "0")) == 0:
            print(f"bench.py: this build runs on one GPU only (asked for {max(args.gpus, world)}); "
                  "the path is single-device and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    import top_reduction_amd as lmh

    sections = set(args.sections.split(","))
    L = lmh.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    timer = Timer(torch)
    steps, warmup, K = args.steps, args.warmup, args.k
    result = {}

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------------
    # headline: prompt-scoring chunk reduce
    # ------------------------------------------------------------------
    rows, V = 256, synth.VOCAB_SCORING
    chunks = []
    for i, dist in enumerate(["normal", "peaked", "gumbel", "normal"]):
        bits, sel = synth.scoring_chunk(7000 + i, dist, K)
        chunks.append((lmh_bf16(torch, bits, dev), torch.from_numpy(sel).to(dev), bits, sel))
        log(f"chunk {i} ({dist}) ready")
    nbytes = rows * V * 2
    ws_size = L.logprob_reduce_workspace_size(rows, V, 128)
    wss = [torch.empty(ws_size, dtype=torch.uint8, device=dev) for _ in chunks]

    def reduce_calls(k):
        outs = []
        fns = []
        for (t, s, _, _), ws in zip(chunks, wss):
            o = (torch.empty(rows, device=dev), torch.empty(rows, device=dev),
                 torch.empty((rows, max(k, 1)), dtype=torch.int32, device=dev),
                 torch.empty((rows, max(k, 1)), device=dev))
            outs.append(o)
            a = (vp(t), lmh.LMH_BF16, rows, V, V, vp(s), k, vp(o[0]), vp(o[1]),
                 vp(o[2]) if k else None, vp(o[3]) if k else None, vp(ws), ws.numel(), None, stream)
            fns.append(lambda a=a: L.logprob_reduce(*a))
        return fns, outs

    fns, _ = reduce_calls(K)
    assert all(f() == 0 for f in fns)
    ms = timer.loop(fns, steps, warmup)
    log(f"reduce K={K}: {ms * 1e3:.1f} us/step")
    red_src = os.path.join(ROOT, "top_reduction_amd", "csrc", "reduce.hip")
    head_src = os.path.join(ROOT, "top_reduction_amd", "csrc", "head.hip")
    row_path = lmh.reduce_row_path(rows, V, K)
    # back-to-back launches of the step's kernel(s): per-step time over the
    # whole timed loop (an event pair around each launch would add its own
    # overhead to every interval)
    t_step = timer.loop_median(fns, steps, warmup)
    achieved = nbytes / (t_step * 1e-3) / 1e9
    if row_path:
        kname = f"k_rowreduce<bf16> (the whole K={K} step in one launch: stream + in-workgroup top-K)"
        tkey = "reduce_row_bf16"
    else:
        kname = f"k_stage1 + k_stage2 (split path, K={K})"
        tkey = None
    log(f"step kernel(s): {t_step * 1e3:.1f} us per step -> {achieved:.0f} GB/s ({kname})")
    roofline = {"bound": "hbm", "kernel": kname,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(tkey, red_src) if tkey else None,
                "bytes_per_launch": nbytes, "launch_us": round(t_step * 1e3, 2)}
    # the split path's streaming kernel alone (what rows that do not fill the
    # CUs evenly go through)
    stage1 = []
    for (t, _, _, _), ws in zip(chunks, wss):
        a = (vp(t), lmh.LMH_BF16, rows, V, V, K, vp(ws), ws.numel(), stream)
        stage1.append(lambda a=a: L.lmh_debug_reduce_stage1(*a))
    t1 = timer.loop_median(stage1, steps, warmup)
    a1 = nbytes / (t1 * 1e-3) / 1e9
    log(f"split-path stage1 alone: {t1 * 1e3:.1f} us per launch -> {a1:.0f} GB/s")
    split_stage1 = {"kernel": "k_stage1<bf16> (split-path streaming pass alone)", "achieved": round(a1, 1),
                    "frac": round(a1 / HBM_PEAK_GBS, 4), "launch_us": round(t1 * 1e3, 2),
                    "traffic": load_traffic("reduce_stage1_bf16", red_src)}

    if "reduce" in sections:
        by_k = {}
        for k in (0, 1, 20, 128):
            f, _ = reduce_calls(k)
            m = timer.loop(f, steps, warmup)
            by_k[str(k)] = {"us": round(m * 1e3, 2), "rows_per_s": round(rows / (m * 1e-3)),
                            "gbps": round(nbytes / (m * 1e-3) / 1e9, 1)}
            log(f"reduce K={k}: {m * 1e3:.1f} us")
        result["reduce_by_k"] = by_k
        # K = -1 (openinfer issue #719, Acceptance criteria): every token's
        # logprob, a [256][248320] fp32 output; bytes = the reduction's read,
        # the second read of the logits and the output write
        full_out = torch.empty((rows, V), device=dev)
        fullf = []
        for (t, s_, _, _), ws in zip(chunks, wss):
            o = (torch.empty(rows, device=dev), torch.empty(rows, device=dev))
            a = (vp(t), lmh.LMH_BF16, rows, V, V, vp(s_), lmh.LMH_K_FULL, vp(o[0]), vp(o[1]), None,
                 vp(full_out), vp(ws), ws.numel(), None, stream)
            fullf.append(lambda a=a, o=o: L.logprob_reduce(*a))
        assert all(f() == 0 for f in fullf)
        m = timer.loop(fullf, max(steps // 4, 10), warmup)
        fb = 2 * nbytes + rows * V * 4
        by_k["-1"] = {"us": round(m * 1e3, 2), "rows_per_s": round(rows / (m * 1e-3)),
                      "gbps": round(fb / (m * 1e-3) / 1e9, 1), "bytes_per_call": fb}
        log(f"reduce K=-1 (full-vocabulary logprobs): {m * 1e3:.1f} us -> {fb / (m * 1e-3) / 1e9:.0f} GB/s")
        del full_out, fullf
        # the same chunks as f16 logits (MTPLX PR #532, Tests: bf16/f16), K = 20
        f16 = [(t.to(torch.float16), s_) for (t, s_, _, _) in chunks]
        fns16 = []
        for (t, s_), ws in zip(f16, wss):
            o = (torch.empty(rows, device=dev), torch.empty(rows, device=dev),
                 torch.empty((rows, K), dtype=torch.int32, device=dev), torch.empty((rows, K), device=dev))
            a = (vp(t), lmh.LMH_F16, rows, V, V, vp(s_), K, vp(o[0]), vp(o[1]), vp(o[2]), vp(o[3]), vp(ws),
                 ws.numel(), None, stream)
            fns16.append(lambda a=a, o=o: L.logprob_reduce(*a))
        assert all(f() == 0 for f in fns16)
        m = timer.loop(fns16, steps, warmup)
        result["reduce_f16"] = {"k": K, "us": round(m * 1e3, 2), "rows_per_s": round(rows / (m * 1e-3)),
                                "gbps": round(nbytes / (m * 1e-3) / 1e9, 1)}
        log(f"reduce f16 K={K}: {m * 1e3:.1f} us")
        del f16, fns16

    # ------------------------------------------------------------------
    # decode rows
    # ------------------------------------------------------------------
    if "decode" in sections:
        bits, sel = synth.decode_logits(7100, sel_mode="uniform")
        base = lmh_bf16(torch, bits, dev)
        copies = [base.clone() for _ in range(32)]
        s = torch.from_numpy(sel).to(dev)
        k = 5
        wsz = L.logprob_reduce_workspace_size(32, synth.VOCAB_QWEN3, k)
        ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
        o = (torch.empty(32, device=dev), torch.empty(32, device=dev),
             torch.empty((32, k), dtype=torch.int32, device=dev), torch.empty((32, k), device=dev))
        f = [lambda t=t: L.logprob_reduce(vp(t), lmh.LMH_BF16, 32, synth.VOCAB_QWEN3,
                                          synth.VOCAB_QWEN3, vp(s), k, vp(o[0]), vp(o[1]), vp(o[2]),
                                          vp(o[3]), vp(ws), ws.numel(), None, stream) for t in copies]
        m = timer.loop(f, steps, warmup)
        result["decode"] = {"workload": "32 x 151936 bf16 decode rows, K=5", "us": round(m * 1e3, 2),
                            "rows_per_s": round(32 / (m * 1e-3)),
                            "gbps": round(32 * synth.VOCAB_QWEN3 * 2 / (m * 1e-3) / 1e9, 1),
                            "path": "split: streaming launch + selection launch"}
        log(f"decode: {m * 1e3:.1f} us")
        # K = 5, 1 and 0: the two launches (logprob_reduce) against the single
        # launch (forced through lmh_debug_reduce_single; the no-workspace
        # entry point takes it at K = 0 only, where it measured faster)
        counters = torch.zeros(4096, dtype=torch.int32, device=dev)
        for kk in (5, 1, 0):
            def two(t, kk=kk):
                return L.logprob_reduce(vp(t), lmh.LMH_BF16, 32, synth.VOCAB_QWEN3, synth.VOCAB_QWEN3, vp(s), kk,
                                        vp(o[0]), vp(o[1]), vp(o[2]) if kk else None,
                                        vp(o[3]) if kk else None, vp(ws), ws.numel(), None, stream)

            def one(t, kk=kk):
                return L.lmh_debug_reduce_single(vp(t), lmh.LMH_BF16, 32, synth.VOCAB_QWEN3, synth.VOCAB_QWEN3,
                                                 vp(s), kk, vp(o[0]), vp(o[1]), vp(o[2]) if kk else None,
                                                 vp(o[3]) if kk else None, vp(ws), ws.numel(), vp(counters), None,
                                                 stream)
            assert two(copies[0]) == 0 and one(copies[0]) == 0
            m2 = timer.loop([lambda t=t: two(t) for t in copies], steps, warmup)
            m1 = timer.loop([lambda t=t: one(t) for t in copies], steps, warmup)
            result["decode"][f"k{kk}"] = {"split_us": round(m2 * 1e3, 2), "single_launch_us": round(m1 * 1e3, 2),
                                          "noalloc_path": "single launch" if kk <= 0 else "split"}
            log(f"decode K={kk}: two launches {m2 * 1e3:.1f} us, single launch {m1 * 1e3:.1f} us")
        del copies

    # ------------------------------------------------------------------
    # selective head (Qwen3-0.6B shape) and the full 2048-row projection
    # ------------------------------------------------------------------
    if "head" in sections:
        d = synth.selective_head_batch(7200)
        hid = lmh_bf16(torch, d["hidden"], dev)
        w = lmh_bf16(torch, d["weight"], dev)
        cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
        T, H = d["hidden"].shape
        Vq = w.shape[0]
        R = 40
        out = torch.empty((R, Vq), device=dev)
        lcu = torch.empty(R + 1, dtype=torch.int32, device=dev)

        def sel_call():
            return L.lmhead_gather_project(vp(hid), lmh.LMH_BF16, T, H, H, vp(w), lmh.LMH_BF16, Vq, H,
                                           vp(cu), R, 0, None, 0, vp(out), lmh.LMH_F32, Vq, vp(lcu),
                                           None, None, stream)

        # three copies of the 311 MB head (933 MB, well above the 256 MB MALL),
        # rotated so that no launch finds its weights in the cache
        wcopies = [w] + [w.clone() for _ in range(2)]

        def sel_kernel(wc):
            return L.lmhead_gather_project(vp(hid), lmh.LMH_BF16, T, H, H, vp(wc), lmh.LMH_BF16, Vq, H,
                                           vp(cu), R, 0, None, 0, vp(out), lmh.LMH_F32, Vq, None,
                                           None, None, stream)
        assert sel_call() == 0
        hs = max(steps // 4, 10)
        m_sel = timer.loop([sel_call], hs, warmup)
        tk = timer.loop_median([lambda wc=wc: sel_kernel(wc) for wc in wcopies], hs, warmup)
        head_bytes = Vq * H * 2 + R * H * 2 + R * Vq * 4
        ach = head_bytes / (tk * 1e-3) / 1e9
        log(f"selective head: call {m_sel * 1e3:.1f} us, kernel {tk * 1e3:.1f} us -> {ach:.0f} GB/s")

        full_idx = torch.arange(2048, dtype=torch.int32, device=dev)
        full = torch.empty((2048, Vq), device=dev)

        def full_call():
            return L.lmhead_gather_project(vp(hid), lmh.LMH_BF16, T, H, H, vp(w), lmh.LMH_BF16, Vq, H,
                                           vp(cu), R, 0, vp(full_idx), 2048, vp(full), lmh.LMH_F32, Vq,
                                           None, None, None, stream)
        assert full_call() == 0
        fs = max(steps // 20, 5)
        tf = timer.loop([full_call], fs, 2)
        flops = 2.0 * 2048 * H * Vq
        tfl = flops / (tf * 1e-3) / 1e12
        log(f"full 2048-row head: {tf * 1e3:.1f} us -> {tfl:.0f} TFLOP/s")
        result["head"] = {
            "workload": "Qwen3-0.6B head: 40 of 81920 packed rows (40 x 2048 prefills), hidden 1024, "
                        "vocab 151936, bf16 in, fp32 logits",
            "selective_ms": round(m_sel, 4), "selective_kernel_us": round(tk * 1e3, 2),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                         "bytes_per_launch": head_bytes, "weight_copies_rotated": len(wcopies),
                         "kernel": "k_head_pipe (k-pipelined weight stream, 16-wave chain per CU)",
                         "traffic": load_traffic("head_pipe_bf16",
                                                 os.path.join(ROOT, "top_reduction_amd", "csrc", "pipe.hip"))},
            "full_2048_ms": round(tf, 4),
            "full_roofline": {"bound": "mfma", "achieved": round(tfl, 1), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tfl / BF16_PEAK_TFLOPS, 4),
                              "traffic": load_traffic("head_tiled_bf16", head_src),
                              "algorithmic_bytes": Vq * H * 2 + 2048 * H * 2 + 2048 * Vq * 4},
        }
        # the same selective and full projections with bf16 logits (the
        # output option of the head; half the logits bytes)
        out16 = torch.empty((R, Vq), dtype=torch.bfloat16, device=dev)
        full16 = torch.empty((2048, Vq), dtype=torch.bfloat16, device=dev)

        def sel16(wc):
            return L.lmhead_gather_project(vp(hid), lmh.LMH_BF16, T, H, H, vp(wc), lmh.LMH_BF16, Vq, H,
                                           vp(cu), R, 0, None, 0, vp(out16), lmh.LMH_BF16, Vq, None,
                                           None, None, stream)

        def full16_call():
            return L.lmhead_gather_project(vp(hid), lmh.LMH_BF16, T, H, H, vp(w), lmh.LMH_BF16, Vq, H,
                                           vp(cu), R, 0, vp(full_idx), 2048, vp(full16), lmh.LMH_BF16, Vq,
                                           None, None, None, stream)
        assert sel16(w) == 0 and full16_call() == 0
        t16 = timer.loop_median([lambda wc=wc: sel16(wc) for wc in wcopies], hs, warmup)
        b16 = Vq * H * 2 + R * H * 2 + R * Vq * 2
        tf16 = timer.loop([full16_call], fs, 2)
        result["head"]["bf16_logits"] = {
            "selective_kernel_us": round(t16 * 1e3, 2),
            "selective_gbps": round(b16 / (t16 * 1e-3) / 1e9, 1),
            "full_2048_ms": round(tf16, 4),
            "full_tflops": round(flops / (tf16 * 1e-3) / 1e12, 1)}
        log(f"bf16 logits: selective {t16 * 1e3:.1f} us, full 2048-row {tf16 * 1e3:.1f} us")
        del out16, full16
        # token bitmask on the 40 selective rows (one segment per row): mask
        # words read once, masked logits written as -inf, nothing else touched
        g = synth.rng(7300)
        words = (Vq + 31) // 32
        masks = [torch.from_numpy(g.integers(0, 2 ** 32, size=(R, words), dtype=np.uint64)
                                  .astype(np.uint32).view(np.int32)).to(dev) for _ in range(4)]
        for m in masks:
            m[:, : words // 2] = 0                           # half the vocabulary fully masked
        outs = [torch.empty((R, Vq), device=dev) for _ in range(4)]

        def mask_call(i):
            return L.lmhead_apply_bitmask(vp(outs[i]), lmh.LMH_F32, R, Vq, Vq, vp(masks[i]), words, None, R,
                                          None, stream)
        assert mask_call(0) == 0
        tm = timer.loop([lambda i=i: mask_call(i) for i in range(4)], hs, warmup)
        result["head"]["bitmask_us"] = round(tm * 1e3, 2)
        log(f"bitmask on 40 x {Vq} fp32 logits: {tm * 1e3:.1f} us")
        del hid, w, wcopies, full, out, outs, masks

    # ------------------------------------------------------------------
    # quantised selective head (Qwen3-0.6B shape, 4- and 8-bit codes, group 64)
    # ------------------------------------------------------------------
    if "headq" in sections:
        d = synth.selective_head_batch(7200, vocab=16)      # the packed hidden rows only
        hid = lmh_bf16(torch, d["hidden"], dev)
        cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
        T, H = d["hidden"].shape
        Vq, R, G = synth.VOCAB_QWEN3, 40, 64
        out = torch.empty((R, Vq), device=dev)
        full_idx = torch.arange(2048, dtype=torch.int32, device=dev)
        full = torch.empty((2048, Vq), device=dev)
        result["headq"] = {}
        for bits in (4, 8):
            qd = synth.quantized_head(7250 + bits, Vq, H, bits, G)
            q = torch.from_numpy(qd["q"].view(np.int32)).to(dev)
            sc = lmh_bf16(torch, qd["scales"], dev)
            bi = lmh_bf16(torch, qd["biases"], dev)
            qld, sld = q.shape[1], sc.shape[1]
            # copies of codes, scales and biases rotated so that together they
            # exceed the 256 MB MALL (4-bit: 4 x 112 MB; 8-bit: 3 x 190 MB)
            ncop = 4 if bits == 4 else 3
            qcopies = [(q, sc, bi)] + [(q.clone(), sc.clone(), bi.clone()) for _ in range(ncop - 1)]

            def sel_q(q=q, sc=sc, bi=bi, qld=qld, sld=sld, bits=bits):
                return L.lmhead_gather_project_q(vp(hid), lmh.LMH_BF16, T, H, H, vp(q), qld, vp(sc),
                                                 vp(bi), sld, bits, G, Vq, vp(cu), R, 0, None, 0,
                                                 vp(out), lmh.LMH_F32, Vq, None, None, None, stream)

            def full_q(q=q, sc=sc, bi=bi, qld=qld, sld=sld, bits=bits):
                return L.lmhead_gather_project_q(vp(hid), lmh.LMH_BF16, T, H, H, vp(q), qld, vp(sc),
                                                 vp(bi), sld, bits, G, Vq, vp(cu), R, 0, vp(full_idx),
                                                 2048, vp(full), lmh.LMH_F32, Vq, None, None, None,
                                                 stream)
            assert sel_q() == 0 and full_q() == 0
            tk = timer.loop_median([lambda c=c: sel_q(*c) for c in qcopies], max(steps // 4, 10), warmup)
            qbytes = Vq * H * bits // 8 + Vq * (H // G) * 4 + R * H * 2 + R * Vq * 4
            ach = qbytes / (tk * 1e-3) / 1e9
            tf = timer.loop([full_q], max(steps // 20, 5), 2)
            tfl = 2.0 * 2048 * H * Vq / (tf * 1e-3) / 1e12
            log(f"quantised head {bits}-bit: selective {tk * 1e3:.1f} us -> {ach:.0f} GB/s; "
                f"full 2048 rows {tf * 1e3:.1f} us -> {tfl:.0f} TFLOP/s")
            result["headq"][f"q{bits}"] = {
                "workload": f"Qwen3-0.6B head, {bits}-bit codes, group {G}, bf16 scale+bias: 40 of "
                            "81920 packed rows, fp32 logits",
                "selective_kernel_us": round(tk * 1e3, 2),
                "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                             "bytes_per_launch": qbytes, "weight_copies_rotated": ncop,
                             "traffic": load_traffic(f"head_stream_q{bits}",
                                                     os.path.join(ROOT, "top_reduction_amd", "csrc",
                                                                  "head.hip"))},
                "full_2048_ms": round(tf, 4),
                "full_roofline": {"bound": "mfma", "achieved": round(tfl, 1),
                                  "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tfl / BF16_PEAK_TFLOPS, 4)},
            }
            del q, sc, bi, qcopies
        del hid, out, full

    # ------------------------------------------------------------------
    # fused head + logprobs (Llama-3-8B shape)
    # ------------------------------------------------------------------
    if "fused" in sections:
        w_np = synth.llama3_head_weight(7300)
        w = lmh_bf16(torch, w_np, dev)
        del w_np
        Vl, H = w.shape
        kk = 20
        fused = {}
        # two copies of the 1.05 GB head, rotated in the mixed-batch loops
        wl = [w, w.clone()]
        for mode in ("mixed", "prompt"):
            d = synth.mixed_batch(7301) if mode == "mixed" else synth.prompt_batch(7302)
            hid = lmh_bf16(torch, d["hidden"], dev)
            cu = torch.from_numpy(d["cu_seqlens"]).to(dev)
            sel = torch.from_numpy(d["selected"]).to(dev)
            ex = None if mode == "mixed" else torch.from_numpy(d["logits_indices"]).to(dev)
            T = hid.shape[0]
            S = cu.numel() - 1
            R = S if ex is None else ex.numel()
            wsz = L.lmhead_logprobs_workspace_size(R, Vl, kk, 256)
            ws = torch.empty(wsz, dtype=torch.uint8, device=dev)
            o = (torch.empty(R, device=dev), torch.empty(R, device=dev),
                 torch.empty((R, kk), dtype=torch.int32, device=dev), torch.empty((R, kk), device=dev))

            def call(wc=w, hid=hid, cu=cu, sel=sel, ex=ex, T=T, S=S, R=R, ws=ws, o=o, nd=d["num_decode"]):
                return L.lmhead_logprobs(vp(hid), lmh.LMH_BF16, T, H, H, vp(wc), lmh.LMH_BF16, Vl, H,
                                         vp(cu), S, nd, None if ex is None else vp(ex),
                                         0 if ex is None else R, vp(sel), kk, vp(o[0]), vp(o[1]),
                                         vp(o[2]), vp(o[3]), None, None, 256, None, vp(ws),
                                         ws.numel(), None, stream)
            assert call() == 0
            n = max(steps // 10, 5)
            fns = [lambda wc=wc: call(wc) for wc in wl] if mode == "mixed" else [call]
            m = timer.loop(fns, n, 3)
            entry = {"ms": round(m, 4), "rows": R, "rows_per_s": round(R / (m * 1e-3))}
            if mode == "mixed":
                entry["workload"] = ("32 decode rows + prefills 512/2048 x4 (10272 tokens), 40 sampled "
                                     "rows, hidden 4096, vocab 128256, K=20")
                wb = Vl * H * 2
                entry["weight_stream_gbps"] = round(wb / (m * 1e-3) / 1e9, 1)
                entry["weight_copies_rotated"] = len(wl)
                # the head stage alone: the same 40 rows projected to fp32 logits
                zout = torch.empty((R, Vl), device=dev)

                def head_only(wc, hid=hid, cu=cu, T=T, S=S, nd=d["num_decode"]):
                    return L.lmhead_gather_project(vp(hid), lmh.LMH_BF16, T, H, H, vp(wc), lmh.LMH_BF16, Vl,
                                                   H, vp(cu), S, nd, None, 0, vp(zout), lmh.LMH_F32, Vl,
                                                   None, None, None, stream)
                assert head_only(w) == 0
                th = timer.loop_median([lambda wc=wc: head_only(wc) for wc in wl], max(n, 10), 3)
                hb = Vl * H * 2 + R * H * 2 + R * Vl * 4
                ha = hb / (th * 1e-3) / 1e9
                entry["head_kernel_us"] = round(th * 1e3, 2)
                entry["head_roofline"] = {"bound": "hbm", "achieved": round(ha, 1), "peak": HBM_PEAK_GBS,
                                          "unit": "GB/s", "frac": round(ha / HBM_PEAK_GBS, 4),
                                          "bytes_per_launch": hb,
                                          "traffic": load_traffic("head_stream_bf16", head_src)}
                log(f"fused mixed head stage alone: {th * 1e3:.1f} us -> {ha:.0f} GB/s")
                del zout
            else:
                entry["workload"] = "one 1024-token prompt, all positions, 256-row chunks, K=20"
                entry["tflops"] = round(2.0 * R * H * Vl / (m * 1e-3) / 1e12, 1)
                entry["reduce_first_pass"] = "tiled head epilogue (per-block partials)"
                # HBM bytes of one 256-row chunk's head launch (counters), against
                # W + hidden rows + fp32 logits + partials and keys
                entry["chunk_head_traffic"] = load_traffic("head_tiled_epilogue_bf16", head_src)
                entry["chunk_head_algorithmic_bytes"] = Vl * H * 2 + 256 * H * 2 + 256 * Vl * 4 + 256 * (-(-Vl // 64)) * 12
                # the same call with the reduction's first pass as its own
                # stream over each chunk's logits
                _, hs = lmh._head_struct(lmh.HeadSpec(w), H)

                def call_unfused(hid=hid, cu=cu, sel=sel, ex=ex, T=T, S=S, R=R, ws=ws, o=o, hs=hs):
                    return L.lmh_debug_logprobs_ex(vp(hid), lmh.LMH_BF16, T, H, H, ctypes.byref(hs), Vl,
                                                   vp(cu), S, 0, vp(ex), R, vp(sel), kk, vp(o[0]), vp(o[1]),
                                                   vp(o[2]), vp(o[3]), None, None, 256, None, None, 0, vp(ws),
                                                   ws.numel(), None, stream, 1)
                assert call_unfused() == 0
                mu = timer.loop([call_unfused], n, 3)
                entry["unfused_ms"] = round(mu, 4)
                log(f"fused prompt with the reduction's own first pass: {mu:.3f} ms")
            fused[mode] = entry
            log(f"fused {mode}: {m:.3f} ms")
            del hid, ws
        result["fused"] = fused
        del w, wl

    # ------------------------------------------------------------------
    # a plain elementwise copy of known size: the reference that scales the
    # HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the kernels above
    # ------------------------------------------------------------------
    if "copycal" in sections:
        src = chunks[0][0]
        dst = torch.empty_like(src)
        for _ in range(max(steps // 10, 5)):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        result["copycal"] = {"kernel": "torch elementwise mul (bf16, in == out size)",
                             "bytes_read": nbytes, "bytes_written": nbytes}
        del dst

    # ------------------------------------------------------------------
    # CPU baseline: the f64 oracle on the scoring chunk
    # ------------------------------------------------------------------
    cpu = None
    if "cpu" in sections:
        import oracle
        # passes over the four chunks in turn until at least 10 s of oracle work
        # (at most 64 passes)
        t0 = time.perf_counter()
        nrows = passes = 0
        while (time.perf_counter() - t0 < 10.0 and passes < 64) or passes == 0:
            bits, sel = chunks[passes % len(chunks)][2], chunks[passes % len(chunks)][3]
            oracle.reduce(bits, sel, K)
            nrows += rows
            passes += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(nrows / dt, 2), "unit": "rows/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{passes} passes over the 256 x 248320 bf16 chunks ({nrows} rows), K={K}, "
                         f"f64 max + exp-sum passes and a full sort per row; {dt:.1f} s"}
        log(f"cpu oracle: {nrows / dt:.1f} rows/s on {cpu['cores']} threads ({dt:.1f} s)")

    line = {
        "metric": METRIC,
        "value": round(rows / (ms * 1e-3)),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prompt-scoring chunk: logprob_reduce over 256 x 248320 bf16 logits, "
                               "K=20, selected ids uniform; 4 seeded chunks (normal, peaked, gumbel, "
                               "normal) rotated",
                   "rows": rows, "vocab": V, "k": K, "input_dtype": "bf16"},
        "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "split_stage1": split_stage1,
        "reduce_path": "one workgroup per row" if row_path else "split (two launches)",
    }
    line.update(result)
    print(json.dumps(line), flush=True)


def lmh_bf16(torch, bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


if __name__ == "__main__":
    main()
