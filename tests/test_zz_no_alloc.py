"""fa_attn_fwd_noalloc (the allocation-free attention call) against fa_attn_fwd through the C
ABI: outputs bit-identical, and within the bf16 tolerance of the oracle, on calls in a row on
one stream -- a 40-head streaming chunk whose 120 items are split into key parts (the parts'
workspace lives in the static array), a smaller bidirectional call with every query kind, and
a smaller split call that reuses the workspace -- plus the host-side errors (unprepared layout,
block map beyond the static array)."""
import ctypes

import numpy as np
import pytest
import torch

import gpu_helpers as G
from frame_aligned_attention_amd import binding as B

TGT, SRC, REF = G.TGT, G.SRC, G.REF


def test_noalloc_host_errors():
    """No GPU needed: both errors are decided on the host before anything is enqueued (the C
    call is made directly, with the default stream, so no device is touched)."""
    io = B.fa_io()
    big = B.make_desc(64, 4096, 64, 128, batch=8, ref_tokens=[64], ref_t0=[0], query_rows=1,
                      block_rows=128)
    L = B.fa_layout_build(big)
    assert B.lib.fa_attn_fwd_noalloc(L.handle, ctypes.byref(io), None) == B.FA_ERR_CAPACITY
    assert b"exceeds the static array" in B.lib.fa_last_error()
    small = B.fa_layout_build(B.make_desc(2, 16, 1, 128, query_rows=1))
    assert B.lib.fa_attn_fwd_noalloc(small.handle, ctypes.byref(io), None) == B.FA_ERR_INVALID
    assert b"fa_layout_prepare" in B.lib.fa_last_error()


def _run(c, noalloc):
    """Like gpu_helpers.run_call, through either entry point, with a prepared layout."""
    tdt = torch.bfloat16
    t = {}
    for k, nm in ((TGT, "q_tgt"), (SRC, "q_src"), (REF, "q_ref")):
        if k in c.kinds() and (k != REF or sum(c.ref_tokens)):
            t[nm] = G.dev(c.q[k], tdt)
    own = (c.cs - c.hist_first) * c.T
    t["k_tgt"], t["v_tgt"] = G.dev(c.k_hist[own:], tdt), G.dev(c.v_hist[own:], tdt)
    t["k_src"], t["v_src"] = G.dev(c.k_src, tdt), G.dev(c.v_src, tdt)
    if sum(c.ref_tokens):
        t["k_ref"], t["v_ref"] = G.dev(c.k_ref, tdt), G.dev(c.v_ref, tdt)
    if c.cache:
        t["k_ring"], t["v_ring"] = G.ring_tensors(c, tdt)
    rows = {TGT: c.C * c.T, SRC: c.C * c.T, REF: sum(c.ref_tokens)}
    outs = {}
    for k in c.kinds():
        if rows[k] == 0:
            continue
        nm = G.KIND_NAMES[k]
        t["o_" + nm] = torch.full((1, rows[k], c.H, c.D), float("nan"), dtype=tdt, device="cuda")
        t["lse_" + nm] = torch.full((1, c.H, rows[k]), float("nan"), dtype=torch.float32,
                                    device="cuda")
        outs[k] = nm
    L = B.fa_layout_build(c.desc(), c.ring_first)
    B.fa_layout_prepare(L)
    if noalloc:
        B.fa_attn_fwd_noalloc(L, B.make_io(t))
    else:
        B.fa_attn_fwd(L, B.make_io(t))
    torch.cuda.synchronize()
    res = {k: (G.host(t["o_" + nm])[0], G.host(t["lse_" + nm])[0]) for k, nm in outs.items()}
    del L
    return res


@pytest.mark.gpu
def test_noalloc_matches_fa_attn_fwd_two_calls():
    calls = [
        ("40-head streaming chunk (T=200, ring wraps, gated reference), ping-pong kernel, "
         "120 items in 2 key parts each",
         G.random_call(71, 200, 3, 40, 128, "bf16", cs=9, window=6, cache=7, ref_tokens=[64, 40],
                       ref_t0=[0, 10], query_rows=1, block_rows=256), 120),
        ("smaller bidirectional call (T=40, F=3, H=2, every query kind), 4-wave kernel",
         G.random_call(72, 40, 3, 2, 128, "bf16", ref_tokens=[24], ref_t0=[1], query_rows=7,
                       block_rows=128), 0),
        ("smaller split call (T=300, F=2, H=1, head_dim 64), ping-pong kernel",
         G.random_call(73, 300, 2, 1, 64, "bf16", ref_tokens=[100], ref_t0=[1], query_rows=3,
                       block_rows=256), 2),
    ]
    for what, c, n_split in calls:
        G.say("case: %s" % what)
        assert B.fa_layout_splits(B.fa_layout_build(c.desc(), c.ring_first))[0] == n_split
        want = _run(c, noalloc=False)
        got = _run(c, noalloc=True)
        assert want.keys() == got.keys()
        for k in want:
            assert np.array_equal(got[k][0], want[k][0]), (what, k, "O differs")
            assert np.array_equal(got[k][1], want[k][1]), (what, k, "LSE differs")
        G.compare_all(c, got, what)
