"""Block map (fa_layout_build) against the oracle's visibility.  CPU only.

For every query row of small layouts -- unaligned frame sizes against the
kernels' 64/128-row tiles, ring wrap, gated references, all three query
kinds -- the keys the block map hands to the kernel (ranges filtered by their
masks) must be exactly the keys the oracle finds visible, each once.  For the
workload-sized layouts the per-row key counts are compared on sampled rows,
and the useful-FLOP totals against the oracle's counts.
"""
import numpy as np
import pytest

import fa_workloads as W
from frame_aligned_attention_amd import binding as B
from oracle import oracle as O

TGT, SRC, REF = O.FAO_TGT, O.FAO_SRC, O.FAO_REF


def ring_slot(g, sink, cap):
    """The ring layout fa.h documents: sink frames keep slots 0 .. sink-1, the others cycle."""
    return g if g < sink else sink + (g - sink) % (cap - sink)


def blockmap_columns(L, d, ring_first, ref_total):
    """{kind: list over rows of the visited key columns} in the oracle's key order
    (target frames 0 .. cs+C-1, then source frames, then reference tokens)."""
    T, C, cs, cap, S = d.tokens_per_frame, d.frames, d.chunk_start, d.cache_frames, d.sink_frames
    nhist = (cs + C) * T
    nsrc = C * T
    present = sorted(set(range(ring_first, cs)) | set(range(min(S, cs))))
    held = {ring_slot(g, S, cap): g for g in present} if cap else {}
    assert len(held) == len(present), "two held frames share a slot"
    n, bm, bn = B.fa_layout_tiles(L)
    out = {}
    for i in range(n):
        (kind, row0, rows), ranges = B.fa_layout_tile(L, i)
        total = {0: C * T, 1: C * T, 2: ref_total}[kind]
        lst = out.setdefault(kind, [None] * total)
        for row in range(row0, row0 + rows):
            cols = []
            fq = row // T
            for seg, beg, end, mask, param in ranges:
                for k in range(beg, end):
                    if mask == B.FA_MASK_SAME_FRAME and k // T != fq:
                        continue
                    if mask == B.FA_MASK_GATE and fq < param:
                        continue
                    if seg == B.FA_SEG_RING:
                        assert k // T in held, "range covers ring slot %d not held" % (k // T)
                        cols.append(held[k // T] * T + k % T)
                    elif seg == B.FA_SEG_TGT:
                        cols.append(cs * T + k)
                    elif seg == B.FA_SEG_SRC:
                        cols.append(nhist + k)
                    else:
                        cols.append(nhist + nsrc + k)
            assert lst[row] is None, "row %d in two tiles" % row
            lst[row] = cols
    return out


def oracle_visibility(d, refs, t0s):
    T, C, cs = d.tokens_per_frame, d.frames, d.chunk_start
    nh, ns, R = (cs + C) * T, C * T, sum(refs)
    nk = nh + ns + R
    eye = np.eye(nk, dtype=np.float32)[:, None, :]
    z = lambda n: np.zeros((n, 1, nk), np.float32)
    g = np.random.default_rng(1)
    k = lambda n: g.standard_normal((n, 1, nk)).astype(np.float32)
    p = O.Problem(T=T, C=C, H=1, D=nk, cs=cs, window=d.window, hist_first=0, ref_tokens=refs,
                  ref_t0=t0s, q_tgt=z(ns), q_src=z(ns), q_ref=z(R), k_hist=k(nh),
                  v_hist=eye[:nh], k_src=k(ns), v_src=eye[nh:nh + ns], k_ref=k(R),
                  v_ref=eye[nh + ns:], sink=d.sink_frames)
    res = O.attn(p)
    return {kind: res[kind][0][:, 0, :] > 0 for kind in res}


SMALL = [
    # frames, T, refs, t0, cs, window, cap, ring_first(-1 default), query_rows, dtype
    (2, 7, [3], [0], 0, 0, 0, -1, 7, B.FA_BF16),
    (3, 24, [16, 5], [0, 2], 0, 0, 0, -1, 7, B.FA_BF16),
    (5, 40, [16], [3], 0, 0, 0, -1, 7, B.FA_F32),
    (1, 64, [16], [0], 0, 0, 0, -1, 7, B.FA_F32),
    (2, 64, [], [], 0, 0, 0, -1, 7, B.FA_F32),
    (3, 50, [20], [0], 9, 4, 5, -1, 1, B.FA_BF16),     # ring wraps: frames 5..8 in slots 0..3
    (3, 50, [20], [0], 12, 4, 5, -1, 3, B.FA_BF16),    # frames 8..11 -> slots 3,4,0,1
    (3, 30, [10, 7], [0, 13], 12, 9, 9, -1, 1, B.FA_BF16),  # gate splits the chunk
    (3, 30, [10, 7], [0, 13], 12, 9, 9, 3, 1, B.FA_LOWBIT),
    (2, 33, [5], [40], 3, 12, 12, 0, 1, B.FA_BF16),    # warm-up: window > history; ref never
    (3, 17, [4], [0], 6, -1, 8, 0, 3, B.FA_BF16),      # all history
    (2, 130, [9], [1], 0, 0, 0, -1, 7, B.FA_BF16),     # tiles across frame boundaries
    (3, 60, [200], [0], 3, 0, 4, -1, 7, B.FA_BF16),    # window 0: no history; 3 frames a tile
    # sink frames (last field): slots 0 .. sink-1 for good, the rest cycle
    (3, 50, [20], [0], 12, 4, 7, -1, 1, B.FA_BF16, 2),  # sink 0,1 + window 8..11 in slots 3..6
    (3, 40, [8], [5], 15, 4, 6, -1, 3, B.FA_BF16, 1),   # window 11..14 wraps in slots 1..5
    (2, 30, [], [], 4, 3, 5, -1, 1, B.FA_BF16, 3),      # sink overlaps the window: all history
    (3, 20, [5], [0], 3, 2, 6, -1, 7, B.FA_F32, 5),     # sink beyond the chunk start
    (2, 64, [16], [0], 10, 0, 3, -1, 1, B.FA_BF16, 2),  # window 0: only the sink frames
    (3, 30, [10], [0], 14, 4, 7, 9, 1, B.FA_LOWBIT, 2), # ring_first given
]


@pytest.mark.parametrize("case", SMALL, ids=[str(i) for i in range(len(SMALL))])
def test_blockmap_equals_oracle_visibility(case):
    F, T, refs, t0s, cs, win, cap, rf, qr, dt, *rest = case
    sink = rest[0] if rest else 0
    hd = 128
    d = B.make_desc(F, T, 1, hd, ref_tokens=refs, ref_t0=t0s, chunk_start=cs, window=win,
                    cache_frames=cap, query_rows=qr, dtype=dt, sink_frames=sink)
    L = B.fa_layout_build(d, rf)
    lo = 0 if win < 0 else max(0, cs - win)
    nlo = max(lo, sink)  # first visible non-sink history frame
    ring_first = rf if rf >= 0 else (nlo if nlo < cs else cs)
    cols = blockmap_columns(L, d, ring_first, sum(refs))
    vis = oracle_visibility(d, refs, t0s)
    kinds = [k for k, bit in ((TGT, 1), (SRC, 2), (REF, 4)) if qr & bit]
    useful = 0
    for kind in kinds:
        want = vis[kind]
        got_rows = cols.get(kind, [])
        assert len(got_rows) == want.shape[0] or want.shape[0] == 0
        for row, c in enumerate(got_rows):
            assert c is not None, "row %d of kind %d in no tile" % (row, kind)
            assert len(c) == len(set(c)), "a key visited twice (kind %d row %d)" % (kind, row)
            got = np.zeros(want.shape[1], bool)
            got[c] = True
            assert np.array_equal(got, want[row]), (kind, row, np.nonzero(got != want[row]))
            useful += len(c)
    st = B.fa_layout_stats(L)
    assert st["useful_pairs"] == useful
    assert st["useful_flops"] == useful * 4 * hd
    assert st["visited_pairs"] >= useful


def test_tile_rows_and_sizes():
    d = B.make_desc(21, 1560, 12, 128, ref_tokens=[1560], ref_t0=[0], query_rows=7, block_rows=128)
    L = B.fa_layout_build(d)
    n, bm, bn = B.fa_layout_tiles(L)
    assert (bm, bn) == (128, 64)
    assert n == 256 + 256 + 13  # 32760 = 255*128 + 120 rows per kind, 1560 reference rows
    (kind, row0, rows), ranges = B.fa_layout_tile(L, 255)
    assert (kind, row0, rows) == (0, 255 * 128, 120)
    # frame boundary tile: rows 1536..1663 cover frames 0 and 1 -> same-frame source range
    (kind, row0, rows), ranges = B.fa_layout_tile(L, 12)
    assert (row0, rows) == (1536, 128)
    assert (B.FA_SEG_SRC, 0, 2 * 1560, B.FA_MASK_SAME_FRAME, 0) in ranges
    (kind, row0, rows), ranges = B.fa_layout_tile(L, 11)
    assert (B.FA_SEG_SRC, 0, 1560, B.FA_MASK_NONE, 0) in ranges


def test_tile_rows_256():
    d = B.make_desc(21, 1560, 12, 128, ref_tokens=[1560], ref_t0=[0], query_rows=7, block_rows=256)
    L = B.fa_layout_build(d)
    n, bm, bn = B.fa_layout_tiles(L)
    assert (bm, bn) == (256, 64)
    assert n == 128 + 128 + 7  # 32760 = 127*256 + 248 rows per kind, 1560 reference rows
    (kind, row0, rows), ranges = B.fa_layout_tile(L, 127)
    assert (kind, row0, rows) == (0, 127 * 256, 248)
    # rows 1280..1535 lie in frame 0; rows 1536..1791 straddle frames 0 and 1
    (kind, row0, rows), ranges = B.fa_layout_tile(L, 5)
    assert (B.FA_SEG_SRC, 0, 1560, B.FA_MASK_NONE, 0) in ranges
    (kind, row0, rows), ranges = B.fa_layout_tile(L, 6)
    assert (B.FA_SEG_SRC, 0, 2 * 1560, B.FA_MASK_SAME_FRAME, 0) in ranges


@pytest.mark.parametrize("wid,split,want,want_splits", [
    (1, B.FA_KEY_SPLIT_AUTO, 256, (0, 0)), (2, B.FA_KEY_SPLIT_AUTO, 256, (0, 0)),
    (3, B.FA_KEY_SPLIT_AUTO, 256, (8, 128)), (3, B.FA_KEY_SPLIT_OFF, 128, (0, 0))])
def test_bf16_block_rows_chosen_by_grid(wid, split, want, want_splits):
    """With block_rows 0 a bf16 layout takes 256-row work items (one 8-wave workgroup per CU)
    unless 128-row items, two to a CU, need clearly fewer rounds over 256 CUs.  The 1560-token
    bidirectional call (3156 vs 6300 items: 13 rounds each; its last round holds cheap
    reference rows, not split) and stream chunk (760 vs 1480: 3 rounds each, the last one
    nearly full) take 256.  The 3600-token chunk has 1032 items = 4 rounds + 8: those 8 are
    cut into 16 key parts each (128 parts on idle CUs, 1/16 of a round), so 256 rows win over
    128-row items' 4 rounds; without the key split it is 5 rounds against 4 and takes 128."""
    w = W.WORKLOADS[wid]
    cs = w.first_cs
    if w.streaming:
        d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.t0_for(cs),
                        chunk_start=cs, window=w.window, cache_frames=w.cache_frames,
                        query_rows=B.FA_Q_TARGET, dtype=B.FA_BF16, key_split=split)
    else:
        d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0,
                        query_rows=7, dtype=B.FA_BF16, key_split=split)
    L = B.fa_layout_build(d)
    _, bm, _ = B.fa_layout_tiles(L)
    assert bm == want
    assert B.fa_layout_splits(L) == want_splits


def frame_intervals(ranges, fq, T):
    """Key intervals per segment that the ranges hand to a row of frame fq, masks applied."""
    out = {}
    for seg, beg, end, mask, param in ranges:
        if mask == B.FA_MASK_SAME_FRAME:
            beg, end = max(beg, fq * T), min(end, (fq + 1) * T)
        elif mask == B.FA_MASK_GATE and fq < param:
            continue
        if beg < end:
            out.setdefault(seg, []).append((beg, end))
    return out


def merged(iv):
    """Sorted union of intervals; fails if two of them overlap (a key handed out twice)."""
    iv = sorted(iv)
    out = []
    for b, e in iv:
        if out:
            assert b >= out[-1][1], "overlap %s" % ((b, e),)
        if out and b == out[-1][1]:
            out[-1] = (out[-1][0], e)
        else:
            out.append((b, e))
    return out


def check_splits(L, T, heads):
    """Every split item's parts: the base tile's rows, ranges inside the base's ranges (same
    segment, mask and parameter), at least 8 key steps each, and between them every key the base
    tile hands to each row exactly once (rows of one frame see the same keys, so per frame).
    Returns (items, parts)."""
    n_split, n_parts = B.fa_layout_splits(L)
    n_tiles, bm, bn = B.fa_layout_tiles(L)
    total = 0
    seen = set()
    for s in range(n_split):
        tile, bh, parts = B.fa_layout_split(L, s)
        assert 0 <= tile < n_tiles and 0 <= bh < heads and bm == 256
        assert (tile, bh) not in seen
        seen.add((tile, bh))
        assert 2 <= len(parts) <= 16
        (kind, row0, rows), base = B.fa_layout_tile(L, tile)
        for (pk, prow0, prows), pr in parts:
            assert (pk, prow0, prows) == (kind, row0, rows)
            steps = 0
            for seg, beg, end, mask, param in pr:
                assert beg < end
                assert any(bs == seg and bb <= beg and end <= be and bm_ == mask and bp == param
                           for bs, bb, be, bm_, bp in base), (seg, beg, end)
                steps += (end - beg + bn - 1) // bn
            assert steps >= 8
        frames = {r // T for r in range(row0, row0 + rows)} if kind < 2 else {0}
        for fq in frames:
            want = frame_intervals(base, fq, T)
            got = {}
            for _, pr in parts:
                for seg, iv in frame_intervals(pr, fq, T).items():
                    got.setdefault(seg, []).extend(iv)
            assert set(got) == set(want), (tile, fq)
            for seg in want:
                assert merged(got[seg]) == merged(want[seg]), (tile, fq, seg)
        total += len(parts)
    assert total == n_parts <= 256
    return n_split, n_parts


SPLIT_CASES = [
    # frames, T, refs, t0, cs, window, cap, query_rows, heads, sink, head_dim
    (3, 300, [200, 150], [0, 13], 12, 4, 6, 7, 2, 1, 128),   # gate inside the chunk, sink frame
    (2, 333, [45], [1], 0, 0, 0, 7, 2, 0, 64),               # bidirectional, ragged frames
    (3, 520, [], [], 9, 6, 9, 1, 3, 0, 128),                  # no reference, ring wraps
    (5, 77, [500], [2], 0, 0, 0, 3, 1, 0, 128),               # many frames per tile
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[str(i) for i in range(len(SPLIT_CASES))])
def test_key_split_parts_cover_tiles(case):
    F, T, refs, t0s, cs, win, cap, qr, H, sink, hd = case
    d = B.make_desc(F, T, H, hd, ref_tokens=refs, ref_t0=t0s, chunk_start=cs, window=win,
                    cache_frames=cap, query_rows=qr, dtype=B.FA_BF16, sink_frames=sink,
                    block_rows=256)
    L = B.fa_layout_build(d)
    n_split, n_parts = check_splits(L, T, H)
    assert n_split > 0 and n_parts >= 2 * n_split
    # the split leaves the block map proper and its counts alone
    d.key_split = B.FA_KEY_SPLIT_OFF
    L0 = B.fa_layout_build(d)
    assert B.fa_layout_splits(L0) == (0, 0)
    assert B.fa_layout_tiles(L0) == B.fa_layout_tiles(L)
    assert B.fa_layout_stats(L0) == B.fa_layout_stats(L)
    for i in range(B.fa_layout_tiles(L)[0]):
        assert B.fa_layout_tile(L0, i) == B.fa_layout_tile(L, i)


def test_key_split_random_layouts():
    """Seeded random bf16 geometries (streaming or bidirectional, references with gates, sink
    frames, all query kinds, 256-row items): wherever the layout splits items, the parts keep
    the invariants of check_splits; the block map proper is the one of the unsplit layout."""
    g = np.random.default_rng(2024)
    split_seen = 0
    for _ in range(60):
        F = int(g.integers(1, 6))
        T = int(g.integers(1, 700))
        nref = int(g.integers(0, 3))
        refs = [int(g.integers(0, 600)) for _ in range(nref)]
        H = int(g.integers(1, 9))
        qr = int(g.integers(1, 8))
        if g.random() < 0.5:
            cs, win, cap, sink = 0, 0, 0, 0
        else:
            sink = int(g.integers(0, 3))
            win = int(g.integers(0, 10))
            cap = win + sink + int(g.integers(0, 3))
            cs = int(g.integers(0, 20))
            if cap == 0:
                cap = 1
        t0s = [int(g.integers(0, cs + F + 2)) for _ in range(nref)]
        d = B.make_desc(F, T, H, 128, ref_tokens=refs, ref_t0=t0s, chunk_start=cs, window=win,
                        cache_frames=cap, query_rows=qr, dtype=B.FA_BF16, sink_frames=sink,
                        block_rows=256)
        try:
            L = B.fa_layout_build(d)
        except B.FaError:
            continue  # a geometry the ring cannot hold
        n_split, _ = check_splits(L, T, H)
        split_seen += n_split > 0
        d.key_split = B.FA_KEY_SPLIT_OFF
        L0 = B.fa_layout_build(d)
        assert B.fa_layout_tiles(L0) == B.fa_layout_tiles(L)
        assert B.fa_layout_stats(L0) == B.fa_layout_stats(L)
    assert split_seen >= 10


def test_key_split_workload_parts():
    """The 3600-token chunk's 8 split items: 16 parts each, one split per (tile, head); their
    scratch is 128 slots of 256 x 129 floats."""
    w, d, L = workload_layout(3)
    assert check_splits(L, w.T, w.H) == (8, 128)
    assert B.fa_layout_workspace_bytes(L) == 128 * 256 * 129 * 4
    assert B.fa_layout_workspace_bytes(workload_layout(2)[2]) == 0


def test_key_split_not_for_128_rows_or_cheap_items():
    # 128-row items: never split
    d = B.make_desc(3, 300, 2, 128, ref_tokens=[200], ref_t0=[0], chunk_start=12, window=4,
                    cache_frames=6, dtype=B.FA_BF16, block_rows=128)
    assert B.fa_layout_splits(B.fa_layout_build(d)) == (0, 0)
    # items under 16 key steps (1024 keys): not worth a split
    d = B.make_desc(2, 150, 2, 128, ref_tokens=[100], ref_t0=[0], query_rows=7, block_rows=256)
    assert B.fa_layout_splits(B.fa_layout_build(d)) == (0, 0)
    # a bad key_split value
    d.key_split = 2
    with pytest.raises(B.FaError):
        B.fa_layout_build(d)


def workload_layout(wid, cs=None):
    w = W.WORKLOADS[wid]
    if w.streaming:
        cs = w.first_cs if cs is None else cs
        d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.t0_for(cs),
                        chunk_start=cs, window=w.window, cache_frames=w.cache_frames,
                        query_rows=B.FA_Q_TARGET, dtype=B.FA_BF16)
    else:
        d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0,
                        query_rows=7, dtype=B.FA_F32 if w.dtype == "f32" else B.FA_BF16)
    return w, d, B.fa_layout_build(d)


def oracle_counts(w, d):
    """Useful pairs per head from the oracle's per-row counts (one row per frame)."""
    cs = d.chunk_start
    p = O.Problem(T=w.T, C=w.C, H=1, D=1, cs=cs, window=d.window if w.streaming else -1,
                  hist_first=0, ref_tokens=w.ref_tokens, ref_t0=list(d.ref_t0)[:len(w.ref_tokens)])
    total = 0
    kinds = [TGT] if w.streaming else [TGT, SRC, REF]
    for kind in kinds:
        if kind == REF:
            total += sum(w.ref_tokens) * O.count(p, REF, 0)
            continue
        for f in range(w.C):
            total += w.T * O.count(p, kind, f * w.T)
    return total


@pytest.mark.parametrize("wid,cs,want_per_head", [
    (0, None, 37120),
    (1, None, 1280073600),
    (2, 57, 124113600),
    (2, 0, None),
    (2, 6, None),
    (3, 12, 570240000),
])
def test_workload_useful_pairs(wid, cs, want_per_head):
    w, d, L = workload_layout(wid, cs)
    st = B.fa_layout_stats(L)
    per_head = st["useful_pairs"] / w.H
    assert per_head == oracle_counts(w, d)
    if want_per_head is not None:
        assert per_head == want_per_head
    # sampled rows: map coverage per row equals the oracle count
    n, bm, bn = B.fa_layout_tiles(L)
    p = O.Problem(T=w.T, C=w.C, H=1, D=1, cs=d.chunk_start,
                  window=d.window if w.streaming else -1, hist_first=0,
                  ref_tokens=w.ref_tokens, ref_t0=list(d.ref_t0)[:len(w.ref_tokens)])
    for i in range(0, n, max(1, n // 23)):
        (kind, row0, rows), ranges = B.fa_layout_tile(L, i)
        for row in (row0, row0 + rows - 1):
            fq = row // w.T
            cnt = 0
            for seg, beg, end, mask, param in ranges:
                if mask == B.FA_MASK_SAME_FRAME:
                    cnt += max(0, min(end, (fq + 1) * w.T) - max(beg, fq * w.T))
                elif mask == B.FA_MASK_GATE:
                    cnt += (end - beg) if fq >= param else 0
                else:
                    cnt += end - beg
            assert cnt == O.count(p, kind, row), (i, row)


def test_stream_layout_sequence():
    """The stream object's layouts over the 20 chunks of the 1560x40-head stream."""
    w = W.WORKLOADS[2]
    d = B.make_desc(w.C, w.T, w.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0, chunk_start=0,
                    window=w.window, cache_frames=w.cache_frames, query_rows=1)
    s = B.Stream(d)
    keys = []
    for cs in W.stream_chunk_starts(w):
        s.seek(cs, max(0, cs - w.cache_frames))
        st = B.fa_layout_stats(s.layout())
        keys.append(st["useful_pairs"] / w.H / (w.C * w.T))
    assert keys[:5] == [7800, 12480, 17160, 21840, 26520]
    assert all(k == 26520 for k in keys[4:])


def test_stream_layout_sequence_with_sink():
    """A stream keeping 2 sink frames beside a 4-frame window (ring of 7 frames): per-row
    history grows to sink + window frames and stays there, and the driver's ring bookkeeping
    (what fa_stream_state reports) matches the ring layout."""
    T, C, win, cap, S = 16, 2, 4, 7, 2
    d = B.make_desc(C, T, 1, 64, chunk_start=0, window=win, cache_frames=cap, query_rows=1,
                    dtype=B.FA_F32, sink_frames=S)
    s = B.Stream(d)
    for cs in range(0, 20, C):
        nf, rf = s.state()
        assert nf == cs
        assert rf == max(0, cs - (cap - S))
        st = B.fa_layout_stats(s.layout())
        hist = len(set(range(max(0, cs - win), cs)) | set(range(min(S, cs))))
        assert st["useful_pairs"] == (hist + C) * T * C * T + C * T * T
        s.seek(cs + C, max(rf, cs + C - (cap - S)))
