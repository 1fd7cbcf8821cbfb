"""Streaming driver (fa_stream_*) on the GPU: a 20-chunk stream of the
1560-token workload (reduced heads) through the ring-buffer KV cache against
the oracle, ring contents, reference injection mid-stream, and
checkpoint/resume."""
import numpy as np
import pytest
import torch

import fa_workloads as W
import gpu_helpers as G
from frame_aligned_attention_amd import binding as B
from oracle import oracle as O

pytestmark = pytest.mark.gpu
TGT = G.TGT


class StreamRun:
    """Drives fa_stream over seeded chunks of workload `wid` with `H` heads."""

    def __init__(self, wid, H, window=None, cache_frames=None, sink=0):
        self.w = W.WORKLOADS[wid]
        if window is not None:
            self.w = W.Workload(**{**self.w.__dict__, "window": window,
                                   "cache_frames": cache_frames})
        w = self.w
        self.H = H
        self.sink = sink
        self.desc = B.make_desc(w.C, w.T, H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0,
                                chunk_start=0, window=w.window, cache_frames=w.cache_frames,
                                query_rows=B.FA_Q_TARGET, dtype=B.FA_BF16, sink_frames=sink)
        self.s = B.Stream(self.desc)
        z = lambda: torch.zeros((1, w.cache_frames * w.T, H, w.D), dtype=torch.bfloat16,
                                device="cuda")
        self.k_ring, self.v_ring = z(), z()
        r = W.ref_tensors(w, H=H)
        self.ref = {"k_ref": G.dev(r["k_ref"]), "v_ref": G.dev(r["v_ref"])}
        self.ref_host = r
        self.k_all, self.v_all = [], []  # host target K/V by chunk

    def chunk_inputs(self, ch):
        x = W.chunk_tensors(self.w, ch, H=self.H)
        return x

    def run_chunk(self, ch):
        w = self.w
        x = self.chunk_inputs(ch)
        t = {"q_tgt": G.dev(x["q_tgt"]), "k_tgt": G.dev(x["k_tgt"]), "v_tgt": G.dev(x["v_tgt"]),
             "k_src": G.dev(x["k_src"]), "v_src": G.dev(x["v_src"]),
             "k_ring": self.k_ring, "v_ring": self.v_ring, **self.ref}
        rows = w.C * w.T
        t["o_tgt"] = torch.empty((1, rows, self.H, w.D), dtype=torch.bfloat16, device="cuda")
        t["lse_tgt"] = torch.empty((1, self.H, rows), dtype=torch.float32, device="cuda")
        self.s.chunk(B.make_io(t))
        torch.cuda.synchronize()
        self.k_all.append(x["k_tgt"])
        self.v_all.append(x["v_tgt"])
        return x, G.host(t["o_tgt"])[0], G.host(t["lse_tgt"])[0]

    def oracle_call(self, ch, x, ref_t0=None):
        w = self.w
        cs = ch * w.C
        lo = 0 if self.sink else max(0, cs - w.window)  # sink frames need the whole history
        c = G.Call(T=w.T, C=w.C, H=self.H, D=w.D, dtype="bf16", cs=cs, window=w.window,
                   cache=w.cache_frames, ref_tokens=list(w.ref_tokens),
                   ref_t0=list(ref_t0 if ref_t0 is not None else w.ref_t0), query_rows=1,
                   hist_first=lo, sink=self.sink)
        kh = np.concatenate(self.k_all[lo // w.C:])
        vh = np.concatenate(self.v_all[lo // w.C:])
        off = (lo - (lo // w.C) * w.C) * w.T
        c.k_hist, c.v_hist = kh[off:], vh[off:]
        c.q = {TGT: x["q_tgt"]}
        c.k_src, c.v_src = x["k_src"], x["v_src"]
        c.k_ref, c.v_ref = self.ref_host["k_ref"], self.ref_host["v_ref"]
        return c


def test_stream_20_chunks_against_oracle():
    G.say("case: 20-chunk stream, T=1560, C=3, window 12, ring 12, H=2")
    run = StreamRun(2, H=2)
    for ch in range(20):
        x, o, lse = run.run_chunk(ch)
        c = run.oracle_call(ch, x)
        if ch in (0, 4, 19):
            p1 = run.oracle_call(ch, x).problem()
            ref = O.attn(p1, kinds=(TGT,))[TGT]
            G.tol_check(o, ref[0], "bf16", "chunk %d all rows" % ch, lse, ref[1],
                        counts=G.row_counts(p1, TGT, np.arange(lse.shape[1]))[None, :])
        else:
            G.compare_sampled(c, {TGT: (o, lse)}, n_rows=24, what="chunk %d" % ch)
    # ring holds frames 48..59 in slots f % 12, bit-exact
    w = run.w
    kr = G.host(run.k_ring)[0]
    for f in range(48, 60):
        s = f % 12
        want = run.k_all[f // 3][(f % 3) * w.T:(f % 3 + 1) * w.T]
        assert np.array_equal(kr[s * w.T:(s + 1) * w.T], want), f
    assert run.s.state() == (60, 48)


def test_stream_checkpoint_resume_bit_identical():
    G.say("case: checkpoint after chunk 7, resume, chunks 8..11 bit-identical")
    a = StreamRun(2, H=1)
    outs = {}
    for ch in range(12):
        _, o, lse = a.run_chunk(ch)
        if ch == 7:
            saved_k, saved_v = a.k_ring.clone(), a.v_ring.clone()
            state = a.s.state()
        if ch >= 8:
            outs[ch] = (o, lse)
    b = StreamRun(2, H=1)
    b.s.seek(*state)
    b.k_ring.copy_(saved_k)
    b.v_ring.copy_(saved_v)
    for ch in range(8, 12):
        _, o, lse = b.run_chunk(ch)
        assert np.array_equal(o, outs[ch][0]) and np.array_equal(lse, outs[ch][1]), ch


def test_stream_reference_injected_mid_stream():
    G.say("case: reference image injected at frame 10 (t0 = 10)")
    run = StreamRun(2, H=1)
    w = run.w
    g = np.random.default_rng(77)
    k2 = W.round_bf16(g.standard_normal((300, 1, w.D), dtype=np.float32))
    v2 = W.round_bf16(g.standard_normal((300, 1, w.D), dtype=np.float32))
    for ch in range(6):
        if ch == 3:  # inject before the chunk at cs = 9: frame 9 must not see it, 10 and 11 must
            run.s.set_refs([1560, 300], [0, 10])
            run.ref = {"k_ref": G.dev(np.concatenate([run.ref_host["k_ref"], k2])),
                       "v_ref": G.dev(np.concatenate([run.ref_host["v_ref"], v2]))}
            run.ref_host = {"k_ref": np.concatenate([run.ref_host["k_ref"], k2]),
                            "v_ref": np.concatenate([run.ref_host["v_ref"], v2])}
            run.w = W.Workload(**{**run.w.__dict__, "ref_tokens": [1560, 300],
                                  "ref_t0": [0, 10]})
        x, o, lse = run.run_chunk(ch)
        if ch >= 2:
            c = run.oracle_call(ch, x)
            G.compare_sampled(c, {TGT: (o, lse)}, n_rows=40, what="inject chunk %d" % ch)


def test_stream_with_sink_frames():
    G.say("case: 12-chunk stream, T=1560, C=3, 2 sink frames + window 6 in an 8-frame ring, H=1")
    run = StreamRun(2, H=1, window=6, cache_frames=8, sink=2)
    w = run.w
    for ch in range(12):
        x, o, lse = run.run_chunk(ch)
        c = run.oracle_call(ch, x)
        if ch == 11:
            p1 = c.problem()
            ref = O.attn(p1, kinds=(TGT,))[TGT]
            G.tol_check(o, ref[0], "bf16", "chunk %d all rows" % ch, lse, ref[1],
                        counts=G.row_counts(p1, TGT, np.arange(lse.shape[1]))[None, :])
        else:
            G.compare_sampled(c, {TGT: (o, lse)}, n_rows=24, what="sink chunk %d" % ch)
    # sink frames 0, 1 in slots 0, 1; frames 30..35 in the cycling slots 2 + (f - 2) % 6
    kr = G.host(run.k_ring)[0]
    for f in (0, 1) + tuple(range(30, 36)):
        s = G.ring_slot(f, 2, 8)
        want = run.k_all[f // 3][(f % 3) * w.T:(f % 3 + 1) * w.T]
        assert np.array_equal(kr[s * w.T:(s + 1) * w.T], want), f
    assert run.s.state() == (36, 30)


APPEND_CASES = [  # dtype, head_dim, batch, T, H, ring frames, sink frames, first frame, frames, pad
    ("bf16", 128, 1, 37, 3, 5, 0, 3, 3, 0),   # frames 3, 4, 5 -> slots 3, 4, 0 (wraps)
    ("bf16", 64, 2, 20, 4, 6, 2, 7, 3, 8),    # 2 sink slots; frames 7..9 -> slots 3..5; padded heads
    ("f32", 128, 2, 9, 2, 4, 1, 0, 4, 0),     # 32 pieces a row; frame 0 into the sink slot
    ("f32", 64, 1, 16, 5, 3, 0, 10, 2, 4),    # frames 10, 11 -> slots 1, 2; padded heads
]


@pytest.mark.parametrize("case", APPEND_CASES,
                         ids=["%s_d%d_b%d" % (c[0], c[1], c[2]) for c in APPEND_CASES])
def test_ring_append_layouts(case):
    """fa_ring_append is pure data movement: the ring after the call equals the ring before with
    each appended frame's tokens in its slot (a sink frame in its own slot, the others cycling
    through the remaining slots), padding between heads untouched, for both element sizes,
    head_dim 64 and 128 and batch 2."""
    dt, D, nb, T, H, cap, sink, f0, nf, pad = case
    G.say("case: ring append %s" % (case,))
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(D + 7 * T + nb)
    full = lambda n: torch.randn((nb, n, H, D + pad), generator=g).to(tdt).cuda()
    rings = [full(cap * T), full(cap * T)]
    chunks = [full(nf * T), full(nf * T)]
    before = [r.clone() for r in rings]
    d = B.make_desc(nf, T, H, D, batch=nb, cache_frames=cap, sink_frames=sink,
                    dtype=B.FA_F32 if dt == "f32" else B.FA_BF16)
    B.fa_ring_append(d, rings[0][..., :D], rings[1][..., :D], chunks[0][..., :D],
                     chunks[1][..., :D], f0, nf)
    torch.cuda.synchronize()
    for r, b0, ch in zip(rings, before, chunks):
        want = b0.clone()
        for fi in range(nf):
            gf = f0 + fi
            slot = gf if gf < sink else sink + (gf - sink) % (cap - sink)
            want[:, slot * T:(slot + 1) * T, :, :D] = ch[:, fi * T:(fi + 1) * T, :, :D]
        assert torch.equal(r, want)
