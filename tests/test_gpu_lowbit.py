"""Low-bit path on the GPU: the quantiser against the oracle's (codes and scales
bit for bit, given the same key mean), and the int8/e4m3 attention against the
fp32 oracle on the unquantised inputs (cosine >= 0.999, max|dO| <= 5e-2), with
a per-channel N(0, 4) key offset to stress the mean smoothing."""
import numpy as np
import pytest
import torch

import fa_workloads as W
import gpu_helpers as G
from frame_aligned_attention_amd import binding as B
from oracle import oracle as O

pytestmark = pytest.mark.gpu
TGT, SRC, REF = G.TGT, G.SRC, G.REF


def lowbit_call(seed, T, C, H, cs=0, window=0, cache=0, refs=(), t0s=(), query_rows=1,
                offset_sd=2.0):
    c = G.random_call(seed, T, C, H, 128, "lowbit", cs=cs, window=window, cache=cache,
                      ref_tokens=refs, ref_t0=t0s, query_rows=query_rows)
    off = np.random.default_rng(seed + 1000).standard_normal((H, 128)).astype(np.float32) * offset_sd
    for name in ("k_hist", "k_src", "k_ref"):
        setattr(c, name, W.round_bf16(getattr(c, name) + off[None]))
    return c


def nblk(n):
    return (n + 127) // 128


class LowbitRun:
    """bf16 inputs of a Call, code/scale buffers, fa_quantize_lowbit + fa_attn_fwd."""

    def __init__(self, c: G.Call):
        self.c = c
        self.desc = c.desc()
        self.L = B.fa_layout_build(self.desc, c.ring_first)
        t = {}
        if TGT in c.kinds():
            t["q_tgt"] = G.dev(c.q[TGT])
        if SRC in c.kinds():
            t["q_src"] = G.dev(c.q[SRC])
        if REF in c.kinds() and sum(c.ref_tokens):
            t["q_ref"] = G.dev(c.q[REF])
        own = (c.cs - c.hist_first) * c.T
        t["k_tgt"], t["v_tgt"] = G.dev(c.k_hist[own:]), G.dev(c.v_hist[own:])
        t["k_src"], t["v_src"] = G.dev(c.k_src), G.dev(c.v_src)
        if sum(c.ref_tokens):
            t["k_ref"], t["v_ref"] = G.dev(c.k_ref), G.dev(c.v_ref)
        if c.cache:
            t["k_ring"], t["v_ring"] = G.ring_tensors(c, torch.bfloat16)
        self.inp = t
        self.codes, self.scales = {}, {}
        for n, x in t.items():
            dt = torch.uint8 if n.startswith("v_") else torch.int8
            self.codes[n] = torch.zeros(x.shape, dtype=dt, device="cuda")
            self.scales[n] = torch.zeros((1, c.H, nblk(x.shape[1])), dtype=torch.float32,
                                         device="cuda")
        self.k_mean = torch.zeros((1, c.H, 128), dtype=torch.float32, device="cuda")
        self.v_absmax = torch.zeros((1, c.H), dtype=torch.float32, device="cuda")
        # outputs; the quantiser writes the per-row smoothing shift into the LSE buffers
        rows = {TGT: c.C * c.T, SRC: c.C * c.T, REF: sum(c.ref_tokens)}
        self.out = {}
        for k in c.kinds():
            if rows[k] == 0:
                continue
            nm = G.KIND_NAMES[k]
            self.out["o_" + nm] = torch.zeros((1, rows[k], c.H, 128), dtype=torch.bfloat16,
                                              device="cuda")
            self.out["lse_" + nm] = torch.zeros((1, c.H, rows[k]), dtype=torch.float32,
                                                device="cuda")

    def quantize(self, mean=None):
        flags = 0
        if mean is not None:
            self.k_mean.copy_(torch.from_numpy(mean).reshape(1, *mean.shape))
            flags = B.FA_QUANT_MEAN_GIVEN
        io_in = B.make_io(self.inp)
        lses = {n: x for n, x in self.out.items() if n.startswith("lse_")}
        io_out = B.make_io({**self.codes, **lses, "k_mean": self.k_mean,
                            "v_absmax": self.v_absmax}, self.scales)
        B.fa_quantize_lowbit(self.L, io_in, io_out, flags)
        torch.cuda.synchronize()

    def attend(self):
        c = self.c
        io = B.make_io({**self.codes, **self.out, "v_absmax": self.v_absmax}, self.scales)
        B.fa_attn_fwd(self.L, io)
        torch.cuda.synchronize()
        return {k: (G.host(self.out["o_" + G.KIND_NAMES[k]])[0],
                    G.host(self.out["lse_" + G.KIND_NAMES[k]])[0])
                for k in c.kinds() if "o_" + G.KIND_NAMES[k] in self.out}


def visible_keys(c: G.Call):
    """Host copies of the key tensors as the quantiser sees them: ring slots out of view zeroed,
    and the token mask of what is in view."""
    segs = {}
    own = (c.cs - c.hist_first) * c.T
    segs["k_tgt"], segs["v_tgt"] = c.k_hist[own:], c.v_hist[own:]
    segs["k_src"], segs["v_src"] = c.k_src, c.v_src
    if sum(c.ref_tokens):
        segs["k_ref"], segs["v_ref"] = c.k_ref, c.v_ref
    masks = {n: np.ones(x.shape[0], bool) for n, x in segs.items()}
    if c.cache:
        cap, T = c.cache, c.T
        for n, src in (("k_ring", c.k_hist), ("v_ring", c.v_hist)):
            r = np.zeros((cap * T, c.H, 128), np.float32)
            m = np.zeros(cap * T, bool)
            for g in range(c.hist_first, c.cs):
                s = g % cap
                i = (g - c.hist_first) * T
                r[s * T:(s + 1) * T] = src[i:i + T]
                m[s * T:(s + 1) * T] = True
            segs[n], masks[n] = r, m
    return segs, masks


QUANT_CASES = [
    # seed, T, C, H, cs, window, cache, refs, t0, query rows
    (41, 50, 3, 2, 9, 4, 5, [20], [0], 1),       # ring wraps; partial 128-blocks everywhere
    (42, 40, 3, 3, 0, 0, 0, [16, 30], [0, 1], 7),  # bidirectional, all query kinds
]


@pytest.mark.parametrize("case", QUANT_CASES, ids=["q%d" % c[0] for c in QUANT_CASES])
def test_quantiser_codes_match_oracle(case):
    seed, T, C, H, cs, win, cap, refs, t0s, qr = case
    G.say("case: quantiser codes %s" % (case,))
    c = lowbit_call(seed, T, C, H, cs, win, cap, refs, t0s, qr)
    run = LowbitRun(c)
    segs, masks = visible_keys(c)
    mean = O.kmean([segs[n][masks[n]] for n in segs if n.startswith("k_")])
    if "k_ring" in segs:  # out-of-view ring tokens: x - m = 0 there, so they do not move absmax
        segs["k_ring"][~masks["k_ring"]] = mean[None]
    run.quantize(mean=mean)
    for n, x in list(segs.items()) + [("q_" + G.KIND_NAMES[k], c.q[k]) for k in c.kinds()
                                      if c.q[k].shape[0]]:
        msk = masks.get(n, np.ones(x.shape[0], bool))
        if n.startswith("v_"):
            codes, scales = O.quant_e4m3(x)
        else:
            codes, scales = O.quant_int8(x, mean=mean if n.startswith("k_") else None)
        got = run.codes[n].cpu().numpy()[0]
        got_s = run.scales[n].cpu().numpy()[0]
        assert np.array_equal(got_s, scales), n
        assert np.array_equal(got[msk], codes[msk].view(got.dtype)), n
    want_absmax = np.max(np.stack([O.quant_e4m3(segs[n])[1].max(1) for n in segs
                                   if n.startswith("v_")]), 0)
    assert np.array_equal(run.v_absmax.cpu().numpy()[0], want_absmax)
    # the device mean (no FA_QUANT_MEAN_GIVEN) agrees with the oracle's to fp32 rounding
    run.quantize(mean=None)
    np.testing.assert_allclose(run.k_mean.cpu().numpy()[0], mean, rtol=2e-5, atol=2e-6)


ATTN_CASES = [
    # seed, T, C, H, cs, window, cache, refs, t0, query rows
    (51, 50, 3, 2, 9, 4, 5, [20], [0], 1),
    (52, 160, 3, 2, 0, 0, 0, [96, 64], [0, 1], 7),  # all query kinds (source rows: 160+ keys)
    (53, 130, 3, 2, 12, 9, 9, [64, 64], [0, 13], 1),  # gate inside the chunk
    (54, 100, 2, 1, 3, 0, 4, [200], [0], 3),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=["a%d" % c[0] for c in ATTN_CASES])
def test_lowbit_attention_against_fp32_oracle(case):
    seed, T, C, H, cs, win, cap, refs, t0s, qr = case
    G.say("case: low-bit attention %s" % (case,))
    c = lowbit_call(seed, T, C, H, cs, win, cap, refs, t0s, qr)
    run = LowbitRun(c)
    run.quantize()
    res = run.attend()
    ref = G.oracle_all(c)
    for k, (o, lse) in res.items():
        G.tol_check(o, ref[k][0], "lowbit", "lowbit %s rows" % G.KIND_NAMES[k], lse, ref[k][1])


def test_lowbit_zero_and_tiny_v_blocks():
    """Keys whose V block is all zero or tiny keep their softmax mass: the row sums run over the
    e4m3 P itself, whatever V's block scale.  The reference image's V is zeroed (two whole
    128-token blocks: about a third of a target row's keys, 256 of 736, and 256 of a source
    row's 416) and the source frames' V is scaled by 1e-10 (block scales near 2^-40).  A row sum
    that dropped the zero-V keys would scale O by ~1.5 and move the LSE by ~ln(2/3) = -0.4; the
    bound holds it to the ordinary low-bit error."""
    case = (61, 160, 2, 2, 0, 0, 0, [256], [0], 3)
    G.say("case: low-bit attention, zero and tiny V blocks %s" % (case,))
    seed, T, C, H, cs, win, cap, refs, t0s, qr = case
    c = lowbit_call(seed, T, C, H, cs, win, cap, refs, t0s, qr)
    c.v_ref = np.zeros_like(c.v_ref)
    c.v_src = W.round_bf16(c.v_src * np.float32(1e-10))
    run = LowbitRun(c)
    run.quantize()
    vs = run.scales["v_ref"].cpu().numpy()
    assert np.all(vs == 0.0), "zero V blocks must get scale 0"
    ss = run.scales["v_src"].cpu().numpy()
    assert np.all((ss > 0) & (ss < 2.0 ** -30)), ss
    res = run.attend()
    ref = G.oracle_all(c)
    for k, (o, lse) in res.items():
        G.tol_check(o, ref[k][0], "lowbit", "lowbit zero/tiny V %s rows" % G.KIND_NAMES[k], lse,
                    ref[k][1])


def lowbit_stream_chunk_call(cs, H):
    """A chunk of the low-bit streaming workload (N(0,4) key offset) with its history."""
    w = W.WORKLOADS[4]
    lo = max(0, cs - w.window)
    c = G.Call(T=w.T, C=w.C, H=H, D=w.D, dtype="lowbit", cs=cs, window=w.window,
               cache=w.cache_frames, ref_tokens=list(w.ref_tokens), ref_t0=list(w.ref_t0),
               query_rows=1, hist_first=lo)
    ks, vs = [], []
    for ch in range(lo // w.C, cs // w.C + 1):
        x = W.chunk_tensors(w, ch, H=H)
        ks.append(x["k_tgt"]); vs.append(x["v_tgt"])
    c.k_hist = np.concatenate(ks)
    c.v_hist = np.concatenate(vs)
    x = W.chunk_tensors(w, cs // w.C, H=H)
    r = W.ref_tensors(w, H=H)
    c.q = {TGT: x["q_tgt"]}
    c.k_src, c.v_src = x["k_src"], x["v_src"]
    c.k_ref, c.v_ref = r["k_ref"], r["v_ref"]
    return c


def test_lowbit_workload_steady_chunk_sampled():
    G.say("case: low-bit workload, steady chunk (cs = 57), 40 heads, sampled rows")
    c = lowbit_stream_chunk_call(57, 40)
    run = LowbitRun(c)
    run.quantize()
    res = run.attend()
    p = c.problem()
    o, lse = res[TGT]
    rows = G.sample_rows(c, TGT, 64)
    heads = [0, 17, 39]
    kk = [TGT] * (len(rows) * len(heads))
    hh = [h for h in heads for _ in rows]
    rr = [int(r) for _ in heads for r in rows]
    ro, rl = O.attn_rows(p, kk, hh, rr)
    go = np.stack([o[r, h] for h, r in zip(hh, rr)])
    gl = np.array([lse[h, r] for h, r in zip(hh, rr)])
    G.tol_check(go, ro, "lowbit", "lowbit steady chunk (sampled %d)" % len(rr), gl, rl)


def test_lowbit_workload_warmup_chunk_full():
    G.say("case: low-bit workload, chunk 2 (cs = 6, ring partly filled), 1 head, every row")
    c = lowbit_stream_chunk_call(6, 1)
    run = LowbitRun(c)
    run.quantize()
    res = run.attend()
    ref = G.oracle_all(c)
    G.tol_check(res[TGT][0], ref[TGT][0], "lowbit", "lowbit chunk 2", res[TGT][1], ref[TGT][1])


def test_lowbit_stream_through_driver():
    """Six chunks of the low-bit workload (2 heads) through fa_stream_layout, fa_quantize_lowbit,
    fa_attn_fwd and fa_stream_advance (the bf16 ring is appended by the driver)."""
    G.say("case: low-bit stream, 6 chunks, 2 heads")
    w = W.WORKLOADS[4]
    H = 2
    d = B.make_desc(w.C, w.T, H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0, chunk_start=0,
                    window=w.window, cache_frames=w.cache_frames, query_rows=1, dtype=B.FA_LOWBIT)
    s = B.Stream(d)
    ring = {n: torch.zeros((1, w.cache_frames * w.T, H, w.D), dtype=torch.bfloat16, device="cuda")
            for n in ("k_ring", "v_ring")}
    r = W.ref_tensors(w, H=H)
    ks, vs = [], []
    for ch in range(6):
        x = W.chunk_tensors(w, ch, H=H)
        t = {"q_tgt": G.dev(x["q_tgt"]), "k_tgt": G.dev(x["k_tgt"]), "v_tgt": G.dev(x["v_tgt"]),
             "k_src": G.dev(x["k_src"]), "v_src": G.dev(x["v_src"]),
             "k_ref": G.dev(r["k_ref"]), "v_ref": G.dev(r["v_ref"]), **ring}
        codes = {n: torch.empty(v.shape, dtype=torch.uint8 if n.startswith("v_") else torch.int8,
                                device="cuda") for n, v in t.items()}
        scales = {n: torch.empty((1, H, nblk(v.shape[1])), dtype=torch.float32, device="cuda")
                  for n, v in t.items()}
        rows = w.C * w.T
        out = {"o_tgt": torch.empty((1, rows, H, w.D), dtype=torch.bfloat16, device="cuda"),
               "lse_tgt": torch.empty((1, H, rows), dtype=torch.float32, device="cuda"),
               "k_mean": torch.empty((1, H, w.D), dtype=torch.float32, device="cuda"),
               "v_absmax": torch.empty((1, H), dtype=torch.float32, device="cuda")}
        L = s.layout()
        B.fa_quantize_lowbit(L, B.make_io(t), B.make_io({**codes, "lse_tgt": out["lse_tgt"],
                                                         "k_mean": out["k_mean"],
                                                         "v_absmax": out["v_absmax"]}, scales))
        B.fa_attn_fwd(L, B.make_io({**codes, **out}, scales))
        s.advance(B.make_io(t))
        torch.cuda.synchronize()
        ks.append(x["k_tgt"]); vs.append(x["v_tgt"])
        cs = ch * w.C
        lo = max(0, cs - w.window)
        c = G.Call(T=w.T, C=w.C, H=H, D=w.D, dtype="lowbit", cs=cs, window=w.window,
                   cache=w.cache_frames, ref_tokens=list(w.ref_tokens), ref_t0=list(w.ref_t0),
                   query_rows=1, hist_first=lo)
        c.k_hist = np.concatenate(ks[lo // w.C:])
        c.v_hist = np.concatenate(vs[lo // w.C:])
        c.q = {TGT: x["q_tgt"]}
        c.k_src, c.v_src, c.k_ref, c.v_ref = x["k_src"], x["v_src"], r["k_ref"], r["v_ref"]
        G.compare_sampled(c, {TGT: (G.host(out["o_tgt"])[0], G.host(out["lse_tgt"])[0])},
                          n_rows=32, what="lowbit stream chunk %d" % ch)
    assert s.state() == (18, 6)


BATCH_CASES = [
    # seed, T, C, H, cs, window, cache, refs, t0, query rows
    (70, 160, 3, 2, 0, 0, 0, [96, 64], [0, 1], 7),   # bidirectional, all query kinds
    (72, 50, 3, 2, 9, 4, 5, [20], [0], 1),           # streaming, the ring wraps
]


@pytest.mark.parametrize("case", BATCH_CASES, ids=["b%d" % c[0] for c in BATCH_CASES])
def test_lowbit_batch2_matches_single_calls(case):
    """Batch 2 through the quantiser and the attention kernel: key means, scales, codes, O and
    LSE of each batch entry equal those of the same inputs run as a batch-1 call (every
    statistic is per (batch, head))."""
    seed, T, C, H, cs, win, cap, refs, t0s, qr = case
    G.say("case: low-bit batch 2 %s" % (case,))
    runs = [LowbitRun(lowbit_call(seed + b, T, C, H, cs, win, cap, refs, t0s, qr)) for b in range(2)]
    single = []
    for r in runs:
        r.quantize()
        single.append(r.attend())
    c0 = runs[0].c
    d = c0.desc()
    d.batch = 2
    L = B.fa_layout_build(d, c0.ring_first)
    cat = lambda f: {n: torch.cat([f(runs[0])[n], f(runs[1])[n]]) for n in f(runs[0])}
    inp = cat(lambda r: r.inp)
    codes = {n: torch.zeros_like(x) for n, x in cat(lambda r: r.codes).items()}
    scales = {n: torch.zeros_like(x) for n, x in cat(lambda r: r.scales).items()}
    out = {n: torch.zeros_like(x) for n, x in cat(lambda r: r.out).items()}
    k_mean = torch.zeros((2, H, 128), dtype=torch.float32, device="cuda")
    v_absmax = torch.zeros((2, H), dtype=torch.float32, device="cuda")
    lses = {n: x for n, x in out.items() if n.startswith("lse_")}
    B.fa_quantize_lowbit(L, B.make_io(inp), B.make_io({**codes, **lses, "k_mean": k_mean,
                                                       "v_absmax": v_absmax}, scales))
    B.fa_attn_fwd(L, B.make_io({**codes, **out, "v_absmax": v_absmax}, scales))
    torch.cuda.synchronize()
    for b, r in enumerate(runs):
        assert torch.equal(k_mean[b], r.k_mean[0]), b
        assert torch.equal(v_absmax[b], r.v_absmax[0]), b
        for n in r.codes:
            assert torch.equal(codes[n][b], r.codes[n][0]), (b, n)
            assert torch.equal(scales[n][b], r.scales[n][0]), (b, n)
        for k, (o, lse) in single[b].items():
            nm = G.KIND_NAMES[k]
            assert np.array_equal(G.host(out["o_" + nm])[b], o), (b, nm)
            assert np.array_equal(G.host(out["lse_" + nm])[b], lse), (b, nm)


RING_Q_CASES = [
    # seed, T, H, ring frames, sink frames, appended (first_frame, frames) in order
    (80, 50, 2, 5, 0, [(0, 3), (3, 3)]),      # second append wraps: frames 3, 4, 5 -> slots 3, 4, 0
    (81, 40, 3, 6, 2, [(0, 3), (3, 3), (6, 3)]),  # sink slots 0, 1; the others cycle through 2..5
]


@pytest.mark.parametrize("case", RING_Q_CASES, ids=["rq%d" % c[0] for c in RING_Q_CASES])
def test_ring_quantize_codes_match_oracle(case):
    """fa_ring_quantize after each fa_ring_append: every 128-token block of the ring that holds
    an appended token has the oracle quantiser's codes and scales for that block's current bf16
    contents (keys less the given mean); every other block keeps what it held."""
    seed, T, H, cap, sink, appends = case
    G.say("case: ring quantiser %s" % (case,))
    g = np.random.default_rng(seed)
    d = B.make_desc(3, T, H, 128, cache_frames=cap, sink_frames=sink, dtype=B.FA_LOWBIT)
    n = cap * T
    ring = {k: torch.zeros((1, n, H, 128), dtype=torch.bfloat16, device="cuda")
            for k in ("k", "v")}
    codes = {"k": torch.full((1, n, H, 128), 99, dtype=torch.int8, device="cuda"),
             "v": torch.full((1, n, H, 128), 99, dtype=torch.uint8, device="cuda")}
    scales = {k: torch.full((1, H, nblk(n)), -1.0, dtype=torch.float32, device="cuda")
              for k in ("k", "v")}
    mean = (g.standard_normal((H, 128)) * 2).astype(np.float32)
    k_mean = torch.from_numpy(mean).reshape(1, H, 128).cuda()
    for f0, nf in appends:
        before = {k: (codes[k].clone(), scales[k].clone()) for k in codes}
        kc = W.round_bf16(g.standard_normal((nf * T, H, 128)).astype(np.float32) * 2 +
                          mean[None])
        vc = W.round_bf16(g.standard_normal((nf * T, H, 128)).astype(np.float32))
        B.fa_ring_append(d, ring["k"], ring["v"], G.dev(kc), G.dev(vc), f0, nf)
        B.fa_ring_quantize(d, ring["k"], ring["v"], codes["k"], codes["v"], scales["k"],
                           scales["v"], k_mean, f0, nf)
        torch.cuda.synchronize()
        touched = set()
        for f in range(f0, f0 + nf):
            s = G.ring_slot(f, sink, cap)
            touched |= set(range(s * T // 128, ((s + 1) * T + 127) // 128))
        kr, vr = G.host(ring["k"])[0], G.host(ring["v"])[0]
        want = {"k": O.quant_int8(kr, mean=mean), "v": O.quant_e4m3(vr)}
        for k in ("k", "v"):
            got_c, got_s = codes[k].cpu().numpy()[0], scales[k].cpu().numpy()[0]
            old_c, old_s = before[k][0].cpu().numpy()[0], before[k][1].cpu().numpy()[0]
            for b in range(nblk(n)):
                sl = slice(b * 128, min(n, (b + 1) * 128))
                if b in touched:
                    assert np.array_equal(got_s[:, b], want[k][1][:, b]), (k, b)
                    assert np.array_equal(got_c[sl], want[k][0][sl].view(got_c.dtype)), (k, b)
                else:
                    assert np.array_equal(got_s[:, b], old_s[:, b]), (k, b, "scale moved")
                    assert np.array_equal(got_c[sl], old_c[sl]), (k, b, "codes moved")


def test_lowbit_stream_with_quantised_ring():
    """Eight chunks of the low-bit workload (2 heads) with the ring kept coded at append time:
    per chunk fa_quantize_lowbit with FA_QUANT_MEAN_GIVEN | FA_QUANT_RING_READY (Q, chunk,
    source, reference only), fa_attn_fwd, fa_stream_advance (bf16 ring) and fa_ring_quantize
    (coded ring), against the fp32 oracle on the unquantised inputs.  The key mean is fixed for
    the stream: the oracle's mean of the reference and first-chunk keys."""
    G.say("case: low-bit stream with a coded ring, 8 chunks, 2 heads")
    w = W.WORKLOADS[4]
    H = 2
    d = B.make_desc(w.C, w.T, H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0, chunk_start=0,
                    window=w.window, cache_frames=w.cache_frames, query_rows=1, dtype=B.FA_LOWBIT)
    s = B.Stream(d)
    n_ring = w.cache_frames * w.T
    ring = {n: torch.zeros((1, n_ring, H, w.D), dtype=torch.bfloat16, device="cuda")
            for n in ("k_ring", "v_ring")}
    ring_codes = {"k_ring": torch.zeros((1, n_ring, H, w.D), dtype=torch.int8, device="cuda"),
                  "v_ring": torch.zeros((1, n_ring, H, w.D), dtype=torch.uint8, device="cuda")}
    ring_scales = {n: torch.zeros((1, H, nblk(n_ring)), dtype=torch.float32, device="cuda")
                   for n in ring_codes}
    r = W.ref_tensors(w, H=H)
    mean = O.kmean([r["k_ref"], W.chunk_tensors(w, 0, H=H)["k_tgt"]])
    k_mean = torch.from_numpy(mean).reshape(1, H, w.D).cuda()
    ks, vs = [], []
    for ch in range(8):
        x = W.chunk_tensors(w, ch, H=H)
        t = {"q_tgt": G.dev(x["q_tgt"]), "k_tgt": G.dev(x["k_tgt"]), "v_tgt": G.dev(x["v_tgt"]),
             "k_src": G.dev(x["k_src"]), "v_src": G.dev(x["v_src"]),
             "k_ref": G.dev(r["k_ref"]), "v_ref": G.dev(r["v_ref"]), **ring}
        codes = {n: torch.empty(v.shape, dtype=torch.uint8 if n.startswith("v_") else torch.int8,
                                device="cuda") for n, v in t.items() if n not in ring}
        scales = {n: torch.empty((1, H, nblk(v.shape[1])), dtype=torch.float32, device="cuda")
                  for n, v in t.items() if n not in ring}
        codes.update(ring_codes)
        scales.update(ring_scales)
        rows = w.C * w.T
        out = {"o_tgt": torch.empty((1, rows, H, w.D), dtype=torch.bfloat16, device="cuda"),
               "lse_tgt": torch.empty((1, H, rows), dtype=torch.float32, device="cuda"),
               "v_absmax": torch.empty((1, H), dtype=torch.float32, device="cuda")}
        L = s.layout()
        B.fa_quantize_lowbit(L, B.make_io(t), B.make_io({**codes, "lse_tgt": out["lse_tgt"],
                                                         "k_mean": k_mean,
                                                         "v_absmax": out["v_absmax"]}, scales),
                             B.FA_QUANT_MEAN_GIVEN | B.FA_QUANT_RING_READY)
        B.fa_attn_fwd(L, B.make_io({**codes, **out}, scales))
        first = s.state()[0]
        s.advance(B.make_io(t))
        B.fa_ring_quantize(d, ring["k_ring"], ring["v_ring"], ring_codes["k_ring"],
                           ring_codes["v_ring"], ring_scales["k_ring"], ring_scales["v_ring"],
                           k_mean, first, w.C)
        torch.cuda.synchronize()
        ks.append(x["k_tgt"]); vs.append(x["v_tgt"])
        cs = ch * w.C
        lo = max(0, cs - w.window)
        c = G.Call(T=w.T, C=w.C, H=H, D=w.D, dtype="lowbit", cs=cs, window=w.window,
                   cache=w.cache_frames, ref_tokens=list(w.ref_tokens), ref_t0=list(w.ref_t0),
                   query_rows=1, hist_first=lo)
        c.k_hist = np.concatenate(ks[lo // w.C:])
        c.v_hist = np.concatenate(vs[lo // w.C:])
        c.q = {TGT: x["q_tgt"]}
        c.k_src, c.v_src, c.k_ref, c.v_ref = x["k_src"], x["v_src"], r["k_ref"], r["v_ref"]
        G.compare_sampled(c, {TGT: (G.host(out["o_tgt"])[0], G.host(out["lse_tgt"])[0])},
                          n_rows=32, what="lowbit coded-ring chunk %d" % ch)
    assert s.state() == (24, 12)
