"""HIP path (libfa.so through the C ABI) against the CPU oracle, element by
element on the same seeded inputs.  Tolerances on O: fp32 max|d| <= 1e-5;
bf16 max|d| <= 1e-2 and mean|d| <= 1e-3; plus LSE bounds (1e-4 fp32; bf16 per
row by its visible-key count, gpu_helpers.lse_tol_bf16) because under N(0,1)
inputs |O| is ~0.01 and an O bound alone would not catch a wrong mask.  The
Q = 0 closed forms at full size are in test_gpu_closed_form.py."""

import numpy as np
import pytest
import torch

import fa_workloads as W
import gpu_helpers as G
from frame_aligned_attention_amd import binding as B

pytestmark = pytest.mark.gpu
TGT, SRC, REF = G.TGT, G.SRC, G.REF


def workload_call(wid, H=None, C=None, T=None) -> G.Call:
    """A bidirectional workload as one call (all query kinds)."""
    w = W.WORKLOADS[wid]
    H, C, T = H or w.H, C or w.C, T or w.T
    x = W.chunk_tensors(w, 0, H=H, T=T, C=C, with_queries_src_ref=True)
    r = W.ref_tensors(w, H=H, with_queries=True)
    c = G.Call(T=T, C=C, H=H, D=w.D, dtype=w.dtype, ref_tokens=list(w.ref_tokens),
               ref_t0=list(w.ref_t0), query_rows=7)
    c.q = {TGT: x["q_tgt"], SRC: x["q_src"], REF: r["q_ref"]}
    c.k_hist, c.v_hist = x["k_tgt"], x["v_tgt"]
    c.k_src, c.v_src = x["k_src"], x["v_src"]
    c.k_ref, c.v_ref = r["k_ref"], r["v_ref"]
    return c


def test_f32_tiny_workload():
    G.say("case: fp32 tiny workload (T=64, F=2, 16 ref tokens, H=2, D=64)")
    c = workload_call(0)
    G.compare_all(c, G.run_call(c), "fp32 tiny")


SMALL = [
    # seed, T, C, H, D, dtype, refs, t0, query_rows
    (1, 7, 2, 2, 128, "bf16", [3], [0], 7),
    (2, 24, 3, 2, 128, "bf16", [16, 5], [0, 2], 7),
    (3, 40, 5, 1, 64, "bf16", [16], [3], 7),
    (4, 130, 2, 3, 128, "bf16", [9], [1], 7),
    (5, 64, 1, 2, 128, "bf16", [], [], 7),
    (6, 200, 3, 2, 128, "bf16", [300, 70], [0, 1], 7),
    (7, 40, 5, 2, 128, "f32", [16], [3], 7),
    (8, 33, 4, 2, 64, "f32", [5, 9], [0, 2], 7),
]


@pytest.mark.parametrize("br", [128, 256], ids=["bm128", "bm256"])
@pytest.mark.parametrize("case", SMALL, ids=["s%d" % c[0] for c in SMALL])
def test_small_shapes(case, br):
    """Each bf16 case through both kernels: 128-row work items (4 waves) and 256-row ones
    (the 8-wave ping-pong kernel)."""
    seed, T, C, H, D, dt, refs, t0s, qr = case
    if dt != "bf16":
        if br == 256:
            pytest.skip("block_rows applies to bf16 only")
        br = 0
    G.say("case: small %s, block_rows %d" % (case, br))
    c = G.random_call(seed, T, C, H, D, dt, ref_tokens=refs, ref_t0=t0s, query_rows=qr,
                      block_rows=br)
    G.compare_all(c, G.run_call(c), "small s%d" % seed)


STREAMS = [
    # seed, T, C, H, D, cs, window, cache, refs, t0
    (11, 50, 3, 2, 128, 9, 4, 5, [20], [0]),         # ring wraps
    (12, 50, 3, 2, 128, 12, 4, 5, [20], [0]),
    (13, 30, 3, 2, 128, 12, 9, 9, [10, 7], [0, 13]),  # t0 gate inside the chunk
    (14, 33, 2, 1, 64, 3, 12, 12, [5], [40]),        # warm-up, reference not yet visible
    (15, 17, 3, 2, 128, 6, -1, 9, [4], [0]),         # all history
    (16, 100, 3, 2, 128, 3, 0, 4, [200], [0]),       # window 0
    # sink frames (last field): frames 0 .. sink-1 stay visible in slots of their own
    (17, 50, 3, 2, 128, 12, 4, 7, [20], [0], 2),     # sink 0, 1 + window 8..11
    (18, 40, 2, 2, 128, 15, 4, 6, [8], [5], 1),      # cycling part wraps
    (19, 64, 3, 1, 128, 10, 0, 3, [16], [0], 2),     # window 0: the sink frames only
    (20, 33, 2, 1, 64, 9, 3, 6, [5], [0], 3),        # head_dim 64
]


@pytest.mark.parametrize("br", [128, 256], ids=["bm128", "bm256"])
@pytest.mark.parametrize("case", STREAMS, ids=["st%d" % c[0] for c in STREAMS])
def test_streaming_calls(case, br):
    seed, T, C, H, D, cs, win, cap, refs, t0s, *rest = case
    G.say("case: streaming %s, block_rows %d" % (case, br))
    c = G.random_call(seed, T, C, H, D, "bf16", cs=cs, window=win, cache=cap, ref_tokens=refs,
                      ref_t0=t0s, query_rows=3, sink=rest[0] if rest else 0, block_rows=br)
    G.compare_all(c, G.run_call(c), "stream st%d" % seed)


@pytest.mark.parametrize("br", [128, 256], ids=["bm128", "bm256"])
def test_bidirectional_reduced(br):
    G.say("case: bidirectional bf16, F=3, T=1560, H=2, all rows, full oracle, block_rows %d" % br)
    c = workload_call(1, H=2, C=3)
    c.block_rows = br
    G.compare_all(c, G.run_call(c), "bidir reduced")


def test_bidirectional_full_size_sampled():
    G.say("case: bidirectional bf16 full size (F=21, T=1560, H=12), sampled rows")
    c = workload_call(1)
    res = G.run_call(c)
    G.compare_sampled(c, res, n_rows=48, heads=[0, 7, 11], what="bidir full")


def stream_call(wid, cs, H=None) -> G.Call:
    """One chunk of a streaming workload with its history (chunk seeds by frame // C)."""
    w = W.WORKLOADS[wid]
    H = H or w.H
    lo = max(0, cs - w.window)
    c = G.Call(T=w.T, C=w.C, H=H, D=w.D, dtype="bf16", cs=cs, window=w.window,
               cache=w.cache_frames, ref_tokens=list(w.ref_tokens), ref_t0=w.t0_for(cs),
               query_rows=1, hist_first=lo)
    ks, vs = [], []
    for ch in range(lo // w.C, cs // w.C + 1):
        x = W.chunk_tensors(w, ch, H=H)
        ks.append(x["k_tgt"]); vs.append(x["v_tgt"])
    first = (lo // w.C) * w.C
    off = (lo - first) * w.T
    c.k_hist = np.concatenate(ks)[off:]
    c.v_hist = np.concatenate(vs)[off:]
    x = W.chunk_tensors(w, cs // w.C, H=H)
    r = W.ref_tensors(w, H=H)
    c.q = {TGT: x["q_tgt"]}
    c.k_src, c.v_src = x["k_src"], x["v_src"]
    c.k_ref, c.v_ref = r["k_ref"], r["v_ref"]
    return c


@pytest.mark.parametrize("br,split,n_split", [(0, B.FA_KEY_SPLIT_AUTO, 8),
                                               (256, B.FA_KEY_SPLIT_OFF, 0),
                                               (128, B.FA_KEY_SPLIT_AUTO, 0)],
                         ids=["auto", "bm256_nosplit", "bm128"])
def test_high_res_chunk_full_size_sampled(br, split, n_split):
    """Full size through the kernel the block map picks (256-row items with the last round's 8
    items split into key parts; head 23's last tile is one of them, and the sample holds its
    rows), through the ping-pong kernel without the split, and through 128-row items."""
    G.say("case: 3600-token chunk at cs=12, window 9, two references (t0 = 0, cs+1), H=24, "
          "block_rows %d, key_split %d" % (br, split))
    c = stream_call(3, 12)
    c.block_rows, c.key_split = br, split
    L = B.fa_layout_build(c.desc(), c.ring_first)
    assert B.fa_layout_splits(L)[0] == n_split
    if n_split:
        assert 23 in [B.fa_layout_split(L, s)[1] for s in range(n_split)]
    res = G.run_call(c)
    G.compare_sampled(c, res, n_rows=64, heads=[0, 23], what="hi-res chunk")


@pytest.mark.parametrize("br", [128, 256], ids=["bm128", "bm256"])
def test_high_res_chunk_reduced_full_oracle(br):
    """H = 1: 43 work items of 256 rows, all in one round, so every one is split into key parts
    (5 each); 128-row items are never split."""
    G.say("case: 3600-token chunk, H=1, every row against the oracle, block_rows %d" % br)
    c = stream_call(3, 12, H=1)
    c.block_rows = br
    n_split = B.fa_layout_splits(B.fa_layout_build(c.desc(), c.ring_first))[0]
    assert n_split == (43 if br == 256 else 0)
    G.compare_all(c, G.run_call(c), "hi-res chunk H=1")


SPLITS = [
    # seed, T, C, H, D, cs, window, cache, refs, t0, query_rows, sink
    (41, 300, 3, 2, 128, 12, 4, 6, [200, 150], [0, 13], 7, 1),  # gate inside the chunk, sink
    (42, 333, 2, 2, 64, 0, 0, 0, [45], [1], 7, 0),              # bidirectional, ragged frames
    (43, 520, 3, 3, 128, 9, 6, 9, [], [], 1, 0),                # no reference, ring wraps
    (44, 77, 5, 1, 128, 0, 0, 0, [500], [2], 3, 0),             # many frames per tile
]


@pytest.mark.parametrize("case", SPLITS, ids=["k%d" % c[0] for c in SPLITS])
def test_key_split_parts(case):
    """256-row items whose keys are split into parts (every item of these one-round grids that
    costs half the largest or more), merged, against the oracle on every row; with a workspace
    of the caller's the output is bit-identical; the same call without the split must agree
    with the oracle too."""
    seed, T, C, H, D, cs, win, cap, refs, t0s, qr, sink = case
    G.say("case: key split %s" % (case,))
    c = G.random_call(seed, T, C, H, D, cs=cs, window=win, cache=cap, ref_tokens=refs,
                      ref_t0=t0s, query_rows=qr, sink=sink, block_rows=256)
    L = B.fa_layout_build(c.desc(), c.ring_first)
    n_split, n_parts = B.fa_layout_splits(L)
    assert n_split > 0 and n_parts >= 2 * n_split
    res = G.run_call(c, layout=L)
    G.compare_all(c, res, "key split")
    # the same call with a workspace of the caller's (fa_io.workspace): bit-identical
    nbytes = B.fa_layout_workspace_bytes(L)
    assert nbytes == n_parts * 256 * (D + 1) * 4
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device="cuda")
    res_ws = G.run_call(c, layout=L, workspace=ws)
    for k in res:
        assert np.array_equal(res_ws[k][0], res[k][0]) and np.array_equal(res_ws[k][1], res[k][1])
    with pytest.raises(B.FaError) as err:  # 4 bytes short: refused before any launch
        G.run_call(c, layout=L, workspace=ws[: (nbytes - 4) // 4])
    assert err.value.status == B.FA_ERR_INVALID
    c.key_split = B.FA_KEY_SPLIT_OFF
    G.compare_all(c, G.run_call(c), "no key split")


def test_key_split_batch2():
    """Batch 2 with split work items (the merge takes batch and head from the item's
    batch*heads index): each batch entry against its own oracle, every row."""
    G.say("case: key split, batch 2 (T=300, C=3, H=2, gated reference)")
    T, C, H, D = 300, 3, 2, 128
    calls = [G.random_call(60 + b, T, C, H, D, "bf16", ref_tokens=[200], ref_t0=[1],
                           query_rows=7, block_rows=256) for b in range(2)]
    d = B.make_desc(C, T, H, D, batch=2, ref_tokens=[200], ref_t0=[1], query_rows=7,
                    block_rows=256)
    L = B.fa_layout_build(d)
    n_split, _ = B.fa_layout_splits(L)
    assert n_split > 0
    assert {B.fa_layout_split(L, s)[1] // H for s in range(n_split)} == {0, 1}  # both batches
    bf = lambda xs: torch.from_numpy(np.stack(xs)).to("cuda").to(torch.bfloat16).contiguous()
    t = {}
    for name, src in (("tgt", lambda c: (c.q[TGT], c.k_hist, c.v_hist)),
                      ("src", lambda c: (c.q[SRC], c.k_src, c.v_src)),
                      ("ref", lambda c: (c.q[REF], c.k_ref, c.v_ref))):
        qs, ks, vs = zip(*[src(c) for c in calls])
        t["q_" + name], t["k_" + name], t["v_" + name] = bf(qs), bf(ks), bf(vs)
        rows = t["q_" + name].shape[1]
        t["o_" + name] = torch.full((2, rows, H, D), float("nan"), dtype=torch.bfloat16,
                                    device="cuda")
        t["lse_" + name] = torch.full((2, H, rows), float("nan"), dtype=torch.float32,
                                      device="cuda")
    B.fa_attn_fwd(L, B.make_io(t))
    torch.cuda.synchronize()
    for b, c in enumerate(calls):
        res = {k: (G.host(t["o_" + nm][b]), G.host(t["lse_" + nm][b]))
               for k, nm in ((TGT, "tgt"), (SRC, "src"), (REF, "ref"))}
        G.compare_all(c, res, "key split batch %d" % b)


# ---------------------------------------------------------------- invariants on the GPU

def test_source_perturbation_is_local():
    """Perturbing source frame j leaves target rows of every other frame bit-identical."""
    G.say("case: source-frame perturbation (bf16, T=200, C=4)")
    c = G.random_call(21, 200, 4, 2, 128, "bf16", ref_tokens=[50], ref_t0=[0], query_rows=3)
    base = G.run_call(c)
    g = np.random.default_rng(5)
    for j in (0, 2):
        c2 = G.random_call(21, 200, 4, 2, 128, "bf16", ref_tokens=[50], ref_t0=[0], query_rows=3)
        c2.k_src[j * 200:(j + 1) * 200] = W.round_bf16(g.standard_normal((200, 2, 128)) * 3)
        c2.v_src[j * 200:(j + 1) * 200] = W.round_bf16(g.standard_normal((200, 2, 128)) * 3)
        res = G.run_call(c2)
        for t in range(4):
            sl = slice(t * 200, (t + 1) * 200)
            same = np.array_equal(res[TGT][0][sl], base[TGT][0][sl]) and np.array_equal(
                res[TGT][1][:, sl], base[TGT][1][:, sl])
            assert same == (t != j), (t, j)


def test_nan_poison_outside_ranges():
    """Ring slots outside the window and output padding hold NaN: results stay finite and
    equal to the clean run."""
    G.say("case: NaN poison in ring slots the block map does not cover")
    c = G.random_call(22, 50, 3, 2, 128, "bf16", cs=12, window=4, cache=7, ref_tokens=[20],
                      ref_t0=[0], query_rows=1)
    clean = G.run_call(c, poison=0.0)
    dirty = G.run_call(c, poison=float("nan"))
    o, lse = dirty[TGT]
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    assert np.array_equal(o, clean[TGT][0]) and np.array_equal(lse, clean[TGT][1])


def test_run_to_run_deterministic():
    G.say("case: determinism (two runs bit-identical)")
    c = workload_call(1, H=2, C=3)
    a = G.run_call(c)
    b = G.run_call(c, out_fill=float("nan"))
    for k in a:
        assert np.array_equal(a[k][0], b[k][0]) and np.array_equal(a[k][1], b[k][1])


@pytest.mark.parametrize("block_rows", [128, 256], ids=["bm128", "bm256"])
def test_strided_and_batched_inputs(block_rows):
    """Q/K/V as views into packed [B, N, 3, H, D] buffers, batch 2: same as separate calls, with
    either bf16 kernel."""
    G.say("case: strided views and batch 2, block_rows %d" % block_rows)
    T, C, H, D = 40, 3, 2, 128
    calls = [G.random_call(30 + b, T, C, H, D, "bf16", ref_tokens=[24], ref_t0=[1],
                           query_rows=7, block_rows=block_rows) for b in range(2)]
    N = C * T
    packed = {}
    for name, src in (("tgt", lambda c: (c.q[TGT], c.k_hist, c.v_hist)),
                      ("src", lambda c: (c.q[SRC], c.k_src, c.v_src)),
                      ("ref", lambda c: (c.q[REF], c.k_ref, c.v_ref))):
        arr = np.stack([np.stack(src(c), 1) for c in calls])  # [B, N, 3, H, D]
        packed[name] = torch.from_numpy(arr).to("cuda").to(torch.bfloat16)
    t = {}
    for name in ("tgt", "src", "ref"):
        p = packed[name]
        t["q_" + name], t["k_" + name], t["v_" + name] = p[:, :, 0], p[:, :, 1], p[:, :, 2]
        rows = p.shape[1]
        t["o_" + name] = torch.zeros((2, rows, H, D), dtype=torch.bfloat16, device="cuda")
        t["lse_" + name] = torch.zeros((2, H, rows), dtype=torch.float32, device="cuda")
    d = B.make_desc(C, T, H, D, batch=2, ref_tokens=[24], ref_t0=[1], query_rows=7,
                    block_rows=block_rows)
    B.fa_attn_fwd(B.fa_layout_build(d), B.make_io(t))
    torch.cuda.synchronize()
    for b, c in enumerate(calls):
        single = G.run_call(c)
        for k, nm in ((TGT, "tgt"), (SRC, "src"), (REF, "ref")):
            assert np.array_equal(G.host(t["o_" + nm][b]), single[k][0]), (b, nm)
            assert np.array_equal(G.host(t["lse_" + nm][b]), single[k][1]), (b, nm)
