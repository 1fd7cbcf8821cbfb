#!/usr/bin/env python3
"""Throughput of the frame-aligned attention hot path on one MI355X.

A step is one streaming chunk of the 1560-token, 40-head workload: the
attention over (ring history in the 12-frame window, the 3-frame chunk, its
3 source frames, the 1560-token reference) followed by the ring append.
Steps walk the 20-chunk stream (chunk i of a step counter k is k mod 20, so a
20-step run covers the warm-up chunks and the steady state); inputs of all 20
chunks are resident in HBM before timing starts.

Prints ONE JSON line.  `value` is useful TFLOP/s (4*head_dim FLOPs per
visible query-key pair) over the timed steps; `roofline` is the attention
kernel against the bf16 MFMA peak, timed with HIP events on the stream the
kernel runs on; `cpu_baseline` is the CPU oracle on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_I8_F8_TOPS = 5000.0    # MI355X dense int8 / fp8 MFMA
METRIC = "frame-aligned attn useful TFLOP/s + ms per streaming chunk, 1 MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_stream1560_h40_traffic.txt")
KERNEL_SRC = os.path.join(ROOT, "frame_aligned_attention_amd", "csrc", "fa_attn_bf16.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_sha():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def traffic_from_profile():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not b or m.group(1) != kernel_sha():
        return None
    return float(b.group(1))


def build_stream_inputs(w, torch, W, B, H=None):
    H = H or w.H
    chunks = []
    rows = w.C * w.T
    r = W.ref_tensors(w, H=H)
    dev = lambda x: torch.from_numpy(x).unsqueeze(0).to("cuda").to(torch.bfloat16).contiguous()
    ref = {"k_ref": dev(r["k_ref"]), "v_ref": dev(r["v_ref"])}
    ring = {n: torch.zeros((1, w.cache_frames * w.T, H, w.D), dtype=torch.bfloat16, device="cuda")
            for n in ("k_ring", "v_ring")}
    o = torch.empty((1, rows, H, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, H, rows), dtype=torch.float32, device="cuda")
    for ch in range(w.chunks):
        x = W.chunk_tensors(w, ch, H=H)
        t = {n: dev(x[n]) for n in ("q_tgt", "k_tgt", "v_tgt", "k_src", "v_src")}
        t.update(ref)
        t.update(ring)
        t["o_tgt"], t["lse_tgt"] = o, lse
        chunks.append((t, B.make_io(t)))
    return chunks


def run_stream_bench(args, torch, W, B):
    w = W.WORKLOADS[2]
    log("bench: generating and uploading %d chunks of %s" % (w.chunks, w.name))
    chunks = build_stream_inputs(w, torch, W, B)
    d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0,
                    chunk_start=0, window=w.window, cache_frames=w.cache_frames,
                    query_rows=B.FA_Q_TARGET, dtype=B.FA_BF16)
    s = B.Stream(d)
    stream = torch.cuda.current_stream()
    n = w.chunks

    # per-chunk layout stats (layouts cached inside the stream object)
    flops = []
    for ch in range(n):
        s.seek(ch * w.C, max(0, ch * w.C - w.cache_frames))
        flops.append(B.fa_layout_stats(s.layout())["useful_flops"])
    s.seek(0, 0)

    def step(k, ev=None):
        ch = k % n
        if ch == 0:
            s.seek(0, 0)
        t, io = chunks[ch]
        L = s.layout()
        if ev is not None:
            ev[0].record(stream)
        B.fa_attn_fwd(L, io, stream)
        if ev is not None:
            ev[1].record(stream)
        s.advance(io, stream)
        if ev is not None:
            ev[2].record(stream)
        return ch

    log("bench: warmup %d steps" % args.warmup)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    log("bench: timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    chs = []
    for k in range(args.steps):
        chs.append(step(args.warmup + k, evs[k]))
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs]
    app_ms = [e[1].elapsed_time(e[2]) for e in evs]
    useful = sum(flops[c] for c in chs)
    steady = [a for a, c in zip(attn_ms, chs) if c >= 4]
    steady_flops = flops[n - 1]
    bytes_chunk = B.fa_layout_stats(s.layout())["bytes"]
    return {
        "w": w, "total_ms": total_ms, "wall_s": wall, "useful": useful, "attn_ms": attn_ms,
        "append_ms": app_ms, "chunks": chs, "flops": flops, "steady": steady,
        "steady_flops": steady_flops, "bytes_steady": bytes_chunk,
    }


def settle(torch, fn, ms=150.0, cap=400):
    """Run fn for about `ms` of GPU time before a timed loop.  Inputs are generated on the host
    just before each workload, the GPU idles meanwhile, and its clocks ramp back up during the
    first calls; a few warm-up calls are not enough to cover that."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(min(cap, int(ms / one) + 1)):
        fn()
    torch.cuda.synchronize()


def time_single_call(wid, torch, W, B, reps=10, sink=0):
    """One-shot workloads (bidirectional 21x1560, 3600-token chunk, the steady chunk of the
    1560-token stream with sink frames): attention call only."""
    w = W.WORKLOADS[wid]
    name = w.name
    dev = lambda x: torch.from_numpy(x).unsqueeze(0).to("cuda").to(torch.bfloat16).contiguous()
    if wid == 1:
        x = W.chunk_tensors(w, 0, with_queries_src_ref=True)
        r = W.ref_tensors(w, with_queries=True)
        t = {n: dev(v) for n, v in {**x, **r}.items()}
        d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0,
                        query_rows=7, dtype=B.FA_BF16)
        rows = {"tgt": w.C * w.T, "src": w.C * w.T, "ref": sum(w.ref_tokens)}
        L = B.fa_layout_build(d)
    else:
        cs = w.first_cs if wid == 3 else (w.chunks - 1) * w.C
        cap = w.cache_frames + sink  # sink frames take slots of their own
        x = W.chunk_tensors(w, cs // w.C)
        r = W.ref_tensors(w)
        t = {n: dev(v) for n, v in {**x, **r}.items()}
        for n in ("k_ring", "v_ring"):
            t[n] = torch.randn((1, cap * w.T, w.H, w.D), device="cuda").to(torch.bfloat16)
        d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.t0_for(cs),
                        chunk_start=cs, window=w.window, cache_frames=cap,
                        query_rows=1, dtype=B.FA_BF16, sink_frames=sink)
        rows = {"tgt": w.C * w.T}
        L = B.fa_layout_build(d, cs - w.window)
        if sink:
            name = "%s + %d sink frames (steady chunk, cs=%d)" % (w.name, sink, cs)
    for nm, n in rows.items():
        t["o_" + nm] = torch.empty((1, n, w.H, w.D), dtype=torch.bfloat16, device="cuda")
        t["lse_" + nm] = torch.empty((1, w.H, n), dtype=torch.float32, device="cuda")
    io = B.make_io(t)
    stream = torch.cuda.current_stream()
    settle(torch, lambda: B.fa_attn_fwd(L, io, stream))
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record(stream)
        B.fa_attn_fwd(L, io, stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    fl = B.fa_layout_stats(L)["useful_flops"]
    med = statistics.median(ms)
    return {"workload": name, "ms_median": round(med, 4), "ms_min": round(min(ms), 4),
            "useful_tflops": round(fl / med / 1e9, 2),
            "mfma_frac": round(fl / med / 1e9 / PEAK_BF16_TFLOPS, 4)}


def time_lowbit_chunk(torch, W, B, reps=10):
    """Low-bit workload, steady chunk (cs = 57), useful ops against the dense int8/fp8 MFMA peak.
    Two flows: (a) the ring kept coded at append time -- per chunk the quantiser codes Q, the
    chunk, its source frames and the reference (FA_QUANT_MEAN_GIVEN | FA_QUANT_RING_READY, the
    stream's fixed key mean), the attention, then the bf16 ring append and fa_ring_quantize of
    the appended frames; (b) everything re-quantised per call (the quantiser also reads the bf16
    ring in view and computes the key mean)."""
    w = W.WORKLOADS[4]
    cs = (w.chunks - 1) * w.C
    dev = lambda x: torch.from_numpy(x).unsqueeze(0).to("cuda").to(torch.bfloat16).contiguous()
    x = W.chunk_tensors(w, cs // w.C)
    r = W.ref_tensors(w)
    t = {n: dev(v) for n, v in {**x, **r}.items()}
    for n in ("k_ring", "v_ring"):
        t[n] = (torch.randn((1, w.cache_frames * w.T, w.H, w.D), device="cuda") * 1.0).to(torch.bfloat16)
    d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0, chunk_start=cs,
                    window=w.window, cache_frames=w.cache_frames, query_rows=1, dtype=B.FA_LOWBIT)
    L = B.fa_layout_build(d)
    codes, scales = {}, {}
    for n, v in t.items():
        codes[n] = torch.empty(v.shape, dtype=torch.uint8 if n.startswith("v_") else torch.int8,
                               device="cuda")
        scales[n] = torch.empty((1, w.H, (v.shape[1] + 127) // 128), dtype=torch.float32,
                                device="cuda")
    rows = w.C * w.T
    out = {"o_tgt": torch.empty((1, rows, w.H, w.D), dtype=torch.bfloat16, device="cuda"),
           "lse_tgt": torch.empty((1, w.H, rows), dtype=torch.float32, device="cuda"),
           "k_mean": torch.empty((1, w.H, w.D), dtype=torch.float32, device="cuda")}
    io_in = B.make_io(t)
    # the attention does not read a V absmax: the quantiser is not asked for one
    io_q = B.make_io({**codes, "lse_tgt": out["lse_tgt"], "k_mean": out["k_mean"]}, scales)
    io_a = B.make_io({**codes, **out}, scales)
    stream = torch.cuda.current_stream()

    def timed(fns):
        settle(torch, lambda: [f() for f in fns])
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
              for _ in range(reps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record(stream)
            for i, f in enumerate(fns):
                f()
                e[i + 1].record(stream)
        torch.cuda.synchronize()
        return [statistics.median([e[i].elapsed_time(e[i + 1]) for e in ev])
                for i in range(len(fns))]

    # (b) everything per call (also establishes the key mean and the ring codes for (a))
    q_ms, a_ms = timed([lambda: B.fa_quantize_lowbit(L, io_in, io_q, 0, stream),
                        lambda: B.fa_attn_fwd(L, io_a, stream)])
    # (a) coded ring: codes of the whole ring from the bf16 ring once, then per chunk
    B.fa_ring_quantize(d, t["k_ring"], t["v_ring"], codes["k_ring"], codes["v_ring"],
                       scales["k_ring"], scales["v_ring"], out["k_mean"], 0, w.cache_frames)
    flags = B.FA_QUANT_MEAN_GIVEN | B.FA_QUANT_RING_READY
    qr_ms, ar_ms, app_ms, rq_ms = timed([
        lambda: B.fa_quantize_lowbit(L, io_in, io_q, flags, stream),
        lambda: B.fa_attn_fwd(L, io_a, stream),
        lambda: B.fa_ring_append(d, t["k_ring"], t["v_ring"], t["k_tgt"], t["v_tgt"], cs, w.C),
        lambda: B.fa_ring_quantize(d, t["k_ring"], t["v_ring"], codes["k_ring"], codes["v_ring"],
                                   scales["k_ring"], scales["v_ring"], out["k_mean"], cs, w.C)])
    ops = B.fa_layout_stats(L)["useful_flops"]
    chunk_ms = qr_ms + ar_ms + app_ms + rq_ms
    return {"workload": w.name + " (steady chunk, cs=57)",
            "quantise_ms": round(qr_ms, 4), "attn_ms": round(ar_ms, 4),
            "ring_append_ms": round(app_ms, 4), "ring_quantise_ms": round(rq_ms, 4),
            "chunk_ms": round(chunk_ms, 4),
            "attn_useful_tops": round(ops / ar_ms / 1e9, 2),
            "attn_frac_of_5000_tops": round(ops / ar_ms / 1e9 / PEAK_I8_F8_TOPS, 4),
            "chunk_useful_tops": round(ops / chunk_ms / 1e9, 2),
            "requantise_every_call": {"quantise_ms": round(q_ms, 4), "attn_ms": round(a_ms, 4)}}


def time_graph_chunk(torch, W, B, lowbit, reps=20):
    """The steady chunk's per-chunk sequence -- (quantise ->) attention -> ring append -- launched
    eagerly and as one captured HIP graph replayed; ms per chunk for both."""
    w = W.WORKLOADS[4 if lowbit else 2]
    cs = (w.chunks - 1) * w.C
    dev = lambda x: torch.from_numpy(x).unsqueeze(0).to("cuda").to(torch.bfloat16).contiguous()
    x = W.chunk_tensors(w, cs // w.C)
    r = W.ref_tensors(w)
    t = {n: dev(v) for n, v in {**x, **r}.items()}
    for n in ("k_ring", "v_ring"):
        t[n] = torch.randn((1, w.cache_frames * w.T, w.H, w.D), device="cuda").to(torch.bfloat16)
    d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0, chunk_start=cs,
                    window=w.window, cache_frames=w.cache_frames, query_rows=1,
                    dtype=B.FA_LOWBIT if lowbit else B.FA_BF16)
    L = B.fa_layout_build(d)
    B.fa_layout_prepare(L)
    rows = w.C * w.T
    out = {"o_tgt": torch.empty((1, rows, w.H, w.D), dtype=torch.bfloat16, device="cuda"),
           "lse_tgt": torch.empty((1, w.H, rows), dtype=torch.float32, device="cuda")}
    if lowbit:
        codes, scales = {}, {}
        for n, v in t.items():
            codes[n] = torch.empty(v.shape, dtype=torch.uint8 if n.startswith("v_") else torch.int8,
                                   device="cuda")
            scales[n] = torch.empty((1, w.H, (v.shape[1] + 127) // 128), dtype=torch.float32,
                                    device="cuda")
        extra = {"k_mean": torch.empty((1, w.H, w.D), dtype=torch.float32, device="cuda")}
        io_in = B.make_io(t)
        io_q = B.make_io({**codes, "lse_tgt": out["lse_tgt"], **extra}, scales)
        io_a = B.make_io({**codes, **out}, scales)
    else:
        io_a = B.make_io({**t, **out})

    def seq():
        if lowbit:
            B.fa_quantize_lowbit(L, io_in, io_q, 0)
        B.fa_attn_fwd(L, io_a)
        B.fa_ring_append(d, t["k_ring"], t["v_ring"], t["k_tgt"], t["v_tgt"], cs, w.C)

    def timed(fn):
        stream = torch.cuda.current_stream()
        settle(torch, fn)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return statistics.median([e[0].elapsed_time(e[1]) for e in ev])

    eager = timed(seq)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    graph = timed(g.replay)
    return {"workload": w.name + " per-chunk sequence (steady chunk, cs=%d)" % cs,
            "kernels": 5 if lowbit else 2, "eager_ms": round(eager, 4),
            "graph_replay_ms": round(graph, 4), "saved_us": round((eager - graph) * 1e3, 1)}


def time_w8a8(torch, W, B, reps=10):
    """Per-block W8A8 QKV projection of a stream chunk: activation quantiser and int8 GEMM;
    useful ops 2*m*n*k against the dense int8 MFMA peak.  torch's bf16 matmul of the same
    shape is timed beside it for context."""
    wl = W.W8A8_QKV
    m, n, k = wl.m, wl.n, wl.k
    x, w = W.linear_tensors(1, m, n, k)
    xd = torch.from_numpy(x).to("cuda").to(torch.bfloat16)
    wd = torch.from_numpy(w).to("cuda").to(torch.bfloat16)
    xq = torch.empty((m, k), dtype=torch.int8, device="cuda")
    wq = torch.empty((n, k), dtype=torch.int8, device="cuda")
    sx = torch.empty((k // 128, m), dtype=torch.float32, device="cuda")
    sw = torch.empty((n // 128, k // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    B.fa_w8a8_quantize_weight(wd, wq, sw)
    wt = wd.t().contiguous()  # w^T [k, n] as a plain contiguous operand

    def timed(fn):
        settle(torch, fn)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        return statistics.median([e[0].elapsed_time(e[1]) for e in ev])

    q_ms = timed(lambda: B.fa_w8a8_quantize_act(xd, xq, sx))
    g_ms = timed(lambda: B.fa_w8a8_gemm(xq, sx, wq, sw, y))
    bf_ms = timed(lambda: torch.mm(xd, wt))
    ops = 2.0 * m * n * k
    return {"workload": wl.name + " (QKV projection of a 1560-token 40-head chunk)",
            "quantise_act_ms": round(q_ms, 4), "gemm_ms": round(g_ms, 4),
            "gemm_tops": round(ops / g_ms / 1e9, 1),
            "gemm_frac_of_5000_tops": round(ops / g_ms / 1e9 / PEAK_I8_F8_TOPS, 4),
            "quantise_plus_gemm_ms": round(q_ms + g_ms, 4),
            "torch_bf16_mm_ms": round(bf_ms, 4)}


def time_prologue(torch, W, B, reps=10):
    """QK prologue on the queries of one chunk of the 1560-token 40-head stream (target and
    source tokens: 9,360 x 40 heads x 128): RMSNorm + RoPE bf16 -> bf16, and fused with the
    low-bit quantiser (-> int8 + block scales); HBM bytes moved against 8 TB/s."""
    n, H, D = 9360, 40, 128
    g = torch.Generator().manual_seed(0)
    x = torch.randn((1, n, H, D), generator=g).to(torch.bfloat16).to("cuda")
    gamma = torch.ones(D, device="cuda")
    p = torch.arange(n)
    pos = torch.stack([57 + (p % 4680) // 1560, (p % 1560) // 52, p % 52], 1).to(torch.int32).cuda()
    y = torch.empty_like(x)
    codes = torch.empty((1, n, H, D), dtype=torch.int8, device="cuda")
    scales = torch.empty((1, H, (n + 127) // 128), dtype=torch.float32, device="cuda")

    def timed(fn):
        settle(torch, fn)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        return statistics.median([e[0].elapsed_time(e[1]) for e in ev])

    t_nr = timed(lambda: B.fa_qk_norm_rope(x, y, gamma, pos))
    t_q = timed(lambda: B.fa_qk_norm_rope_quant(x, codes, scales, gamma, pos, False))
    nb = n * H * D * 2
    return {"workload": "qk-prologue-9360x40x128 (queries of a 1560-token 40-head chunk)",
            "norm_rope_ms": round(t_nr, 4), "norm_rope_gbs": round(2 * nb / t_nr / 1e6, 1),
            "norm_rope_quant_ms": round(t_q, 4),
            "norm_rope_quant_gbs": round(1.5 * nb / t_q / 1e6, 1),
            "hbm_frac": round(2 * nb / t_nr / 1e6 / 8000.0, 3)}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(W, budget_s=15.0):
    """The oracle, as it stands, on a deterministic sample of the steady chunk (chunk 19) of the
    1560-token 40-head stream.  The sample is a fixed sequence of batches -- 8 of the 40 heads
    (0, 5, ..., 35); for each head the frame-boundary rows first, then every 4th row -- taken in
    that order until the whole sequence is done or `budget_s` seconds of oracle time have passed
    (so the CPU leg stays bounded on a slow host); each row sees its 26,520 keys.  The oracle's
    useful-FLOP rate on it, scaled to the chunk's 2.542 TFLOP, gives the oracle time per steady
    chunk.  (The survey's fuller plan -- every chunk for 4 heads plus all heads of chunks 0, 3
    and 19 -- is several minutes of CPU time; this bench keeps its CPU leg to seconds.)"""
    import numpy as np
    from oracle import oracle as O
    w = W.WORKLOADS[2]
    heads = list(range(0, w.H, 5))
    H = len(heads)
    cs = (w.chunks - 1) * w.C
    lo = max(0, cs - w.window)
    ks, vs = [], []
    for ch in range(lo // w.C, cs // w.C + 1):
        x = W.chunk_tensors(w, ch)
        ks.append(x["k_tgt"][:, heads]); vs.append(x["v_tgt"][:, heads])
    x = W.chunk_tensors(w, cs // w.C)
    r = W.ref_tensors(w)
    p = O.Problem(T=w.T, C=w.C, H=H, D=w.D, cs=cs, window=w.window, hist_first=lo,
                  ref_tokens=w.ref_tokens, ref_t0=w.ref_t0, q_tgt=x["q_tgt"][:, heads],
                  k_hist=np.concatenate(ks), v_hist=np.concatenate(vs), k_src=x["k_src"][:, heads],
                  v_src=x["v_src"][:, heads], k_ref=r["k_ref"][:, heads], v_ref=r["v_ref"][:, heads],
                  q_src=np.zeros((0, H, w.D), np.float32), q_ref=np.zeros((0, H, w.D), np.float32))
    rows_total = w.C * w.T
    bounds = sorted({0, rows_total - 1} | {f * w.T + d for f in range(1, w.C) for d in (-1, 0)})
    order = bounds + [rw for rw in range(0, rows_total, 4) if rw not in bounds]
    keys = O.count(p, O.FAO_TGT, 0)
    done, spent = 0, 0.0
    for hi in range(H):
        for b0 in range(0, len(order), 256):
            batch = order[b0:b0 + 256]
            t0 = time.perf_counter()
            O.attn_rows(p, [O.FAO_TGT] * len(batch), [hi] * len(batch), batch)
            spent += time.perf_counter() - t0
            done += len(batch)
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    fl = done * keys * 4 * w.D
    rate = fl / spent
    chunk_flops = w.H * rows_total * keys * 4 * w.D
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": O.threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "ms_per_steady_chunk": round(chunk_flops / rate * 1e3, 1),
            "sample": "steady chunk (chunk 19) of the 1560-token 40-head stream: %d query rows "
                      "(heads 0,5,..,35 in turn; per head the frame-boundary rows, then every 4th "
                      "row; stopped after %.1f s), %d visible keys each, %.3g useful FLOP"
                      % (done, spent, keys, fl)}


def summarize_rocprof(prefix, out_dir):
    """Writes the committed rocprofv3 summaries from the CSV output of the commands below
    (run with this same bench.py): kernel trace statistics, and HBM traffic of the attention
    kernel per launch from FETCH_SIZE / WRITE_SIZE, each scaled by what the counter reads for the
    plain 1 GiB device copy that --copy-check runs in the same process."""
    import csv
    import glob
    import fa_workloads as W
    from frame_aligned_attention_amd import binding as B
    cmd = "python bench.py --steps 20 --warmup 20 --no-cpu-baseline --no-extra --copy-check 1024"
    trace_cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d %s_trace -o trace -- %s"
                 % (prefix, cmd))
    stats = list(csv.DictReader(open(glob.glob(prefix + "_trace/*kernel_stats.csv")[0])))
    lines = ["# rocprofv3 kernel statistics: 1560-token 40-head stream, 20 warm-up + 20 timed "
             "chunks (attention + ring append each), after a 1 GiB calibration copy",
             "# command: " + trace_cmd,
             "# kernel source sha256[:16] (fa_attn_bf16.hip): " + kernel_sha(),
             "%-44s %6s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
    for r in stats[:8]:
        name = r["Name"]
        name = name if len(name) <= 44 else name[:41] + "..."
        lines.append("%-44s %6s %12.1f %12.1f %12.1f" % (
            name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3))
    os.makedirs(out_dir, exist_ok=True)
    open(os.path.join(out_dir, "attn_bf16_stream1560_h40_trace.txt"), "w").write(
        "\n".join(lines) + "\n")

    def per_dispatch(counter):
        rows = list(csv.DictReader(open(glob.glob(prefix + "_%s/*counter_collection.csv"
                                                  % counter)[0])))
        d = {}
        for r in rows:
            k = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            d[k] = d.get(k, 0.0) + float(r["Counter_Value"])
        return sorted(d.items())
    res = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        items = per_dispatch(counter)
        copy = max(v for (i, n), v in items if "copyBuffer" in n or "copy" in n.lower())
        factor = (1 << 30) / (copy * 1024.0)
        attn = [v for (i, n), v in items if "attn_bf16" in n]
        kname = sorted({n for (i, n), v in items if "attn_bf16" in n})
        timed = attn[20:40]  # 20 warm-up launches, then the 20 timed ones
        res[counter] = (factor, sum(timed) / len(timed) * 1024.0 * factor, copy)
    w = W.WORKLOADS[2]
    d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0, chunk_start=0,
                    window=w.window, cache_frames=w.cache_frames, query_rows=B.FA_Q_TARGET)
    s = B.Stream(d)
    alg = []
    for ch in range(w.chunks):
        s.seek(ch * w.C, max(0, ch * w.C - w.cache_frames))
        alg.append(B.fa_layout_stats(s.layout())["bytes"])
    alg_mean = sum(alg) / len(alg)
    hbm = res["FETCH_SIZE"][1] + res["WRITE_SIZE"][1]
    text = [
        "# HBM traffic of the bf16 attention kernel (%s), per launch," % ", ".join(kname),
        "# mean over the 20 timed chunks of the 1560-token 40-head stream (chunks 0..19: warm-up",
        "# and steady state)",
        "# commands (one rocprofv3 pass per counter):",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d %s_FETCH_SIZE -o pmc -- %s" % (prefix, cmd),
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d %s_WRITE_SIZE -o pmc -- %s" % (prefix, cmd),
        "# calibration: the same runs first copy 1 GiB device to device (--copy-check 1024);",
        "#   FETCH_SIZE read %.0f KiB for it -> scale %.4f; WRITE_SIZE read %.0f KiB -> scale %.4f"
        % (res["FETCH_SIZE"][2], res["FETCH_SIZE"][0], res["WRITE_SIZE"][2], res["WRITE_SIZE"][0]),
        "kernel_source_sha256_16: %s" % kernel_sha(),
        "fetch_bytes_per_launch: %.4e" % res["FETCH_SIZE"][1],
        "write_bytes_per_launch: %.4e" % res["WRITE_SIZE"][1],
        "hbm_bytes_per_launch: %.4e" % hbm,
        "algorithmic_bytes_per_launch: %.4e" % alg_mean,
        "traffic_over_algorithmic: %.3f" % (hbm / alg_mean),
    ]
    open(os.path.join(out_dir, "attn_bf16_stream1560_h40_traffic.txt"), "w").write(
        "\n".join(text) + "\n")
    print("\n".join(lines + text))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other bf16 workloads")
    ap.add_argument("--summarize-rocprof", metavar="PREFIX",
                    help="write profiles/ summaries from rocprofv3 CSVs under PREFIX_{trace,"
                         "FETCH_SIZE,WRITE_SIZE} and exit")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (calibrates HBM counters)")
    ap.add_argument("--only", choices=["bidir", "hires", "lowbit", "w8a8"],
                    help="time that one workload alone (for profiler runs) and print its line")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the attention "
              "would shard by head). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import fa_workloads as W
    from frame_aligned_attention_amd import binding as B
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_check:
        n = args.copy_check * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log("bench: copy check %d MiB read + %d MiB written" % (args.copy_check, args.copy_check))
        del a, b
    if args.only:
        fn = {"bidir": lambda: time_single_call(1, torch, W, B),
              "hires": lambda: time_single_call(3, torch, W, B),
              "lowbit": lambda: time_lowbit_chunk(torch, W, B),
              "w8a8": lambda: time_w8a8(torch, W, B)}[args.only]
        print(json.dumps(fn()), flush=True)
        return
    res = run_stream_bench(args, torch, W, B)
    w = res["w"]
    value = res["useful"] / res["total_ms"] / 1e9  # TFLOP/s
    ms_step = res["total_ms"] / args.steps
    attn_mean = statistics.mean(res["attn_ms"])
    useful_per_launch = res["useful"] / args.steps
    achieved = useful_per_launch / attn_mean / 1e9
    traffic = traffic_from_profile()
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s: 20-chunk stream, 3 frames x 1560 tokens per chunk, window 12 "
                               "frames, ring 12 frames, 1560 reference tokens, 40 heads, head_dim "
                               "128, batch 1; step = attention + ring append of one chunk" % w.name,
                   "tokens_per_frame": w.T, "chunk_frames": w.C, "heads": w.H,
                   "head_dim": w.D, "window": w.window, "ring_frames": w.cache_frames,
                   "ref_tokens": sum(w.ref_tokens)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "attn_ms_mean": round(attn_mean, 4),
        "attn_ms_steady_median": round(statistics.median(res["steady"]), 4) if res["steady"] else None,
        "steady_chunk_tflops": round(res["steady_flops"] / statistics.median(res["steady"]) / 1e9, 2)
        if res["steady"] else None,
        "append_ms_mean": round(statistics.mean(res["append_ms"]), 4),
        "steady_chunk_hbm_gbs": round(res["bytes_steady"] / statistics.median(res["steady"]) / 1e6, 1)
        if res["steady"] else None,
        "wall_s": round(res["wall_s"], 3),
    }
    if not args.no_extra:
        log("bench: other bf16 workloads")
        out["other_workloads"] = [time_single_call(1, torch, W, B), time_single_call(3, torch, W, B),
                                  time_lowbit_chunk(torch, W, B),
                                  time_single_call(2, torch, W, B, sink=3),
                                  time_graph_chunk(torch, W, B, False),
                                  time_graph_chunk(torch, W, B, True),
                                  time_w8a8(torch, W, B),
                                  time_prologue(torch, W, B)]
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline (fixed sample of the steady chunk)")
        out["cpu_baseline"] = cpu_baseline(W)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
