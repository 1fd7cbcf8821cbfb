"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each pin_* takes an oracle library handle (so tests/test_oracle_mutants.py can
run the same pins against deliberately broken builds of the oracle) and
raises AssertionError when the oracle disagrees.  Every pin uses tiny shapes.

What pins what:
  golden masks      hand-written visibility matrices (tests/golden/mask_*.txt)
                    -> every visibility rule, including the t0 gate and window
  dense brute force torch scaled_dot_product_attention in float64 with a dense
                    boolean mask from token labels -> whole predicate + softmax
  F = 1             plain unmasked attention (library routine)
  two keys          closed form sigmoid -> the scale, base e, LSE formula
  Q = 0             O = mean of the visible V, LSE = ln(#visible) exactly
  rows == full      the single-row entry point returns the full call's slices bit for bit
  V = 1             rows of probabilities sum to one
  perturbation      each "only" of the rule: bit-identical outputs
  permutation       key order inside a frame does not matter
  split / merge     LSE-weighted merge of two disjoint key sets
  streaming         cs = 0 streaming == bidirectional; window >= cs == all
  sink              sink 0 == plain window; sink reaching the window == all history;
                    exactly the sink and window frames matter
  smoothing         subtracting a per-channel vector from all keys is exact
  quantiser         hand-derived codes, round-trip bound, torch float8_e4m3fn
  W8A8              hand-derived block codes, torch round; integer matmul (numpy), per-block
                    scale weighting, closed-form quantisation error bound
  norm + RoPE       numpy RMSNorm at position 0, norm kept, relative positions, hand-derived
                    single-pair rotations on each axis
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from oracle import oracle as O

TGT, SRC, REF = O.FAO_TGT, O.FAO_SRC, O.FAO_REF
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------- helpers

def rand_problem(seed, T, C, H, D, cs=0, window=-1, hist_first=None, ref_tokens=(),
                 ref_t0=(), bf16=False, sink=0):
    g = np.random.default_rng(seed)
    if hist_first is None:
        hist_first = 0

    def n(*shape):
        x = g.standard_normal(size=shape).astype(np.float32)
        if bf16:
            x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
        return x

    nh = (cs + C - hist_first) * T
    R = int(sum(ref_tokens))
    return O.Problem(T=T, C=C, H=H, D=D, cs=cs, window=window, hist_first=hist_first,
                     ref_tokens=list(ref_tokens), ref_t0=list(ref_t0),
                     q_tgt=n(C * T, H, D), q_src=n(C * T, H, D), q_ref=n(R, H, D),
                     k_hist=n(nh, H, D), v_hist=n(nh, H, D), k_src=n(C * T, H, D),
                     v_src=n(C * T, H, D), k_ref=n(R, H, D), v_ref=n(R, H, D), sink=sink)


def clone(p, **kw):
    d = {k: getattr(p, k) for k in ("T", "C", "H", "D", "cs", "window", "hist_first",
                                    "ref_tokens", "ref_t0", "scale", "sink")}
    for k in ("q_tgt", "q_src", "q_ref", "k_hist", "v_hist", "k_src", "v_src", "k_ref", "v_ref"):
        a = getattr(p, k)
        d[k] = None if a is None else a.copy()
    d.update(kw)
    return O.Problem(**d)


def key_labels(p):
    """(kind, frame, image) per key, keys ordered hist | source | reference."""
    kinds, frames, imgs = [], [], []
    for g in range(p.hist_first, p.cs + p.C):
        kinds += [TGT] * p.T; frames += [g] * p.T; imgs += [-1] * p.T
    for g in range(p.cs, p.cs + p.C):
        kinds += [SRC] * p.T; frames += [g] * p.T; imgs += [-1] * p.T
    for r, n in enumerate(p.ref_tokens):
        kinds += [REF] * n; frames += [-1] * n; imgs += [r] * n
    return np.array(kinds), np.array(frames), np.array(imgs)


def dense_mask(p, qkind):
    """Dense boolean visibility [rows, keys] built from labels (a second formulation)."""
    kk, kf, ki = key_labels(p)
    rows = p.rows(qkind)
    if qkind == REF:
        return np.broadcast_to(kk == REF, (rows, kk.size)).copy()
    qf = p.cs + np.arange(rows) // p.T
    lo = 0 if p.window < 0 else max(0, p.cs - p.window)
    t0 = np.array(list(p.ref_t0) + [0])[ki]
    same_src = (kk == SRC)[None] & (kf[None] == qf[:, None])
    ref_ok = (kk == REF)[None] & (qf[:, None] >= t0[None])
    if qkind == SRC:
        return same_src | ref_ok
    tgt_ok = ((kk == TGT) & ((kf >= lo) | (kf < p.sink)) & (kf < p.cs + p.C))[None]
    return tgt_ok | same_src | ref_ok


def dense_reference(p, qkind):
    kv = [a for a in (p.k_hist, p.k_src, p.k_ref) if a is not None and a.size]
    vv = [a for a in (p.v_hist, p.v_src, p.v_ref) if a is not None and a.size]
    K = torch.from_numpy(np.concatenate(kv, 0)).double().permute(1, 0, 2)
    V = torch.from_numpy(np.concatenate(vv, 0)).double().permute(1, 0, 2)
    q = {TGT: p.q_tgt, SRC: p.q_src, REF: p.q_ref}[qkind]
    Q = torch.from_numpy(q).double().permute(1, 0, 2)
    mask = torch.from_numpy(dense_mask(p, qkind))
    scale = p.scale if p.scale is not None else 1.0 / math.sqrt(p.D)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask[None],
                                                         scale=scale)
    s = (Q @ K.transpose(1, 2)) * scale
    s = s.masked_fill(~mask[None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(1, 0, 2).numpy(), lse.numpy()


def close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, "%s: max rel err %.3g > %.3g" % (what, err, tol)


def read_golden(path):
    meta, mat, rows = {}, [], None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("# layout:"):
                for kv in line[len("# layout:"):].split():
                    k, v = kv.split("=")
                    meta[k] = [int(x) for x in v.split(",") if x != ""] if k.startswith(
                        "ref_") else int(v)
            elif line.startswith("rows:"):
                t = line.split()
                rows = {t[1]: int(t[2]), t[3]: int(t[4]), t[5]: int(t[6])}
            elif line and not line.startswith("#"):
                mat.append([int(x) for x in line.split()])
    return meta, rows, np.array(mat, dtype=bool)


# ---------------------------------------------------------------------------- pins

def pin_golden_masks(lib):
    files = sorted(f for f in os.listdir(GOLDEN) if f.startswith("mask_"))
    assert files
    for fn in files:
        meta, rows, want = read_golden(os.path.join(GOLDEN, fn))
        p0 = O.Problem(T=meta["T"], C=meta["C"], H=1, D=1, cs=meta["cs"], window=meta["window"],
                       hist_first=meta["hist_first"], ref_tokens=meta["ref_tokens"],
                       ref_t0=meta["ref_t0"], sink=meta.get("sink", 0))
        nk = (p0.cs + p0.C - p0.hist_first) * p0.T * 1 + p0.C * p0.T + sum(p0.ref_tokens)
        D = max(nk, 2)
        eye = np.eye(nk, D, dtype=np.float32)[:, None, :]
        nh = (p0.cs + p0.C - p0.hist_first) * p0.T
        ns = p0.C * p0.T
        R = sum(p0.ref_tokens)
        g = np.random.default_rng(7)
        z = lambda n: np.zeros((n, 1, D), np.float32)
        k = lambda n: g.standard_normal((n, 1, D)).astype(np.float32)
        p = O.Problem(T=p0.T, C=p0.C, H=1, D=D, cs=p0.cs, window=p0.window,
                      hist_first=p0.hist_first, ref_tokens=p0.ref_tokens, ref_t0=p0.ref_t0,
                      q_tgt=z(ns), q_src=z(ns), q_ref=z(R), k_hist=k(nh), v_hist=eye[:nh],
                      k_src=k(ns), v_src=eye[nh:nh + ns], k_ref=k(R), v_ref=eye[nh + ns:],
                      sink=p0.sink)
        res = O.attn(p, lib=lib)
        got = np.concatenate([res[TGT][0][:, 0, :nk], res[SRC][0][:, 0, :nk],
                              res[REF][0][:, 0, :nk]], 0) > 0
        assert got.shape == want.shape, fn
        assert np.array_equal(got, want), "%s: visibility differs\n%s" % (fn, got.astype(int))


LAYOUTS = [
    # (T, C, cs, window, hist_first, ref_tokens, ref_t0[, sink])
    (1, 1, 0, -1, 0, (), ()),
    (7, 2, 0, -1, 0, (3,), (0,)),
    (7, 3, 0, -1, 0, (3, 5), (0, 2)),
    (24, 5, 0, -1, 0, (16,), (0,)),
    (5, 3, 3, 3, 0, (4,), (0,)),
    (5, 3, 9, 3, 6, (4, 2), (0, 10)),
    (3, 3, 21, 12, 9, (2, 2), (5, 22)),
    (4, 2, 3, 12, 0, (3,), (4,)),
    (4, 2, 9, 0, 9, (), ()),
    (2, 3, 6, -1, 0, (2,), (7,)),
    (3, 2, 9, 3, 0, (2,), (10,), 2),
    (2, 3, 12, 4, 0, (), (), 5),
    (3, 2, 4, 1, 0, (2,), (0,), 9),
]


def layout_args(lay):
    T, C, cs, w, hf, rt, r0, *rest = lay
    return dict(T=T, C=C, cs=cs, window=w, hist_first=hf, ref_tokens=rt, ref_t0=r0,
                sink=rest[0] if rest else 0)


def pin_bruteforce(lib):
    for i, lay in enumerate(LAYOUTS):
        a = layout_args(lay)
        p = rand_problem(100 + i, a["T"], a["C"], 2, 8, a["cs"], a["window"], a["hist_first"],
                         a["ref_tokens"], a["ref_t0"], sink=a["sink"])
        res = O.attn(p, lib=lib)
        for kind in (TGT, SRC, REF):
            if p.rows(kind) == 0:
                continue
            o_ref, lse_ref = dense_reference(p, kind)
            close(res[kind][0], o_ref, 2e-6, "O kind %d layout %d" % (kind, i))
            close(res[kind][1], lse_ref, 2e-6, "LSE kind %d layout %d" % (kind, i))


def pin_f1_full_attention(lib):
    p = rand_problem(5, 6, 1, 3, 16, ref_tokens=(4, 3), ref_t0=(0, 0))
    res = O.attn(p, lib=lib)
    K = torch.from_numpy(np.concatenate([p.k_hist, p.k_src, p.k_ref])).double().permute(1, 0, 2)
    V = torch.from_numpy(np.concatenate([p.v_hist, p.v_src, p.v_ref])).double().permute(1, 0, 2)
    Q = torch.from_numpy(p.q_tgt).double().permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V).permute(1, 0, 2).numpy()
    close(res[TGT][0], o, 2e-6, "F=1 target rows vs plain attention")


def pin_two_keys(lib):
    # One target frame of one token, one source token, no reference; D = 2.
    # s1 = (q.k1)/sqrt(2) = sqrt(2), s2 = 0  ->  o = sigma(sqrt 2) v1 + (1 - sigma(sqrt 2)) v2
    f = lambda *v: np.array(v, np.float32).reshape(1, 1, -1)
    p = O.Problem(T=1, C=1, H=1, D=2, q_tgt=f(1, 0), q_src=f(0, 0), q_ref=None,
                  k_hist=f(2, 0), v_hist=f(1, 0), k_src=f(0, 1), v_src=f(0, 1))
    res = O.attn(p, kinds=(TGT,), lib=lib)
    sig = 1.0 / (1.0 + math.exp(-math.sqrt(2.0)))
    close(res[TGT][0][0, 0], [sig, 1.0 - sig], 1e-7, "two-key O")
    close(res[TGT][1][0, 0], math.sqrt(2.0) + math.log1p(math.exp(-math.sqrt(2.0))), 1e-7,
          "two-key LSE")


def pin_large_scores(lib):
    # Scores 0, 750 and 760 (beyond exp's double range): the softmax is still defined,
    # o = (e^-10 v2 + v3) / (1 + e^-10) up to e^-760, and lse = 760 + ln(1 + e^-10).
    f = lambda *v: np.array(v, np.float32).reshape(-1, 1, 2)
    r2 = math.sqrt(2.0)
    p = O.Problem(T=1, C=1, H=1, D=2, q_tgt=f(1, 0), q_src=f(0, 0),
                  k_hist=f(0, 1), v_hist=f(5, 5),
                  k_src=f(750 * r2, 0), v_src=f(1, 0),
                  ref_tokens=[1], ref_t0=[0], q_ref=f(0, 0), k_ref=f(760 * r2, 0), v_ref=f(0, 1))
    res = O.attn(p, kinds=(TGT,), lib=lib)
    w = math.exp(-10.0)
    close(res[TGT][0][0, 0], [w / (1 + w), 1 / (1 + w)], 1e-6, "large-score O")
    close(res[TGT][1][0, 0], 760.0 + math.log1p(w), 1e-6, "large-score LSE")


def expected_count(p, kind, row):
    """Closed-form visible-key count of one row."""
    if kind == REF:
        return sum(p.ref_tokens)
    f = p.cs + row // p.T
    refs = sum(n for n, t0 in zip(p.ref_tokens, p.ref_t0) if f >= t0)
    if kind == SRC:
        return p.T + refs
    lo = 0 if p.window < 0 else max(0, p.cs - p.window)
    sink_only = max(0, min(p.sink, lo))  # sink frames below the window
    return (p.cs + p.C - lo + sink_only) * p.T + p.T + refs


def visible_mean(p, kind, row, h):
    """Mean of the visible V rows by slicing the segments (another formulation)."""
    if kind == REF:
        return p.v_ref[:, h].astype(np.float64).mean(0)
    f = p.cs + row // p.T
    parts = []
    if kind == TGT:
        lo = 0 if p.window < 0 else max(0, p.cs - p.window)
        sink_end = min(p.sink, lo)
        if sink_end > 0:
            parts.append(p.v_hist[(0 - p.hist_first) * p.T:(sink_end - p.hist_first) * p.T, h])
        parts.append(p.v_hist[(lo - p.hist_first) * p.T:, h])
    parts.append(p.v_src[(f - p.cs) * p.T:(f - p.cs + 1) * p.T, h])
    off = 0
    for n, t0 in zip(p.ref_tokens, p.ref_t0):
        if f >= t0:
            parts.append(p.v_ref[off:off + n, h])
        off += n
    return np.concatenate(parts).astype(np.float64).mean(0)


def pin_q_zero(lib):
    for i, lay in enumerate(LAYOUTS):
        a = layout_args(lay)
        p = rand_problem(200 + i, a["T"], a["C"], 2, 8, a["cs"], a["window"], a["hist_first"],
                         a["ref_tokens"], a["ref_t0"], sink=a["sink"])
        for name in ("q_tgt", "q_src", "q_ref"):
            setattr(p, name, np.zeros_like(getattr(p, name)))
        res = O.attn(p, lib=lib)
        for kind in (TGT, SRC, REF):
            for row in range(p.rows(kind)):
                n = expected_count(p, kind, row)
                assert O.count(p, kind, row, lib=lib) == n
                for h in range(p.H):
                    close(res[kind][1][h, row], math.log(n), 1e-7, "Q=0 LSE")
                    close(res[kind][0][row, h], visible_mean(p, kind, row, h), 1e-6, "Q=0 O")


def pin_rows_match_full(lib):
    """fa_oracle_attn_rows (the entry point behind every sampled full-size check) returns, for
    each (kind, head, row) it is asked for, exactly the slice fa_oracle_attn writes for that
    row: same O bits, same LSE bits, over every layout (sink and gated ones included).  H = 3
    and rows both above and below H make a swapped head/row index visible."""
    g = np.random.default_rng(11)
    for i, lay in enumerate(LAYOUTS):
        a = layout_args(lay)
        p = rand_problem(300 + i, a["T"], a["C"], 3, 8, a["cs"], a["window"], a["hist_first"],
                         a["ref_tokens"], a["ref_t0"], sink=a["sink"])
        full = O.attn(p, lib=lib)
        kk, hh, rr = [], [], []
        for kind in (TGT, SRC, REF):
            n = p.rows(kind)
            if n == 0:
                continue
            rows = list(range(n)) if n <= 8 else sorted(set(g.integers(0, n, 8).tolist()) |
                                                          {0, n - 1})
            for r in rows:
                for h in range(p.H):
                    kk.append(kind); hh.append(h); rr.append(r)
        order = g.permutation(len(kk))
        kk, hh, rr = [kk[j] for j in order], [hh[j] for j in order], [rr[j] for j in order]
        o, lse = O.attn_rows(p, kk, hh, rr, lib=lib)
        for j, (kind, h, r) in enumerate(zip(kk, hh, rr)):
            assert np.array_equal(o[j], full[kind][0][r, h]), ("rows O", i, kind, h, r)
            assert np.array_equal(lse[j], full[kind][1][h, r]), ("rows LSE", i, kind, h, r)


def pin_ones_v(lib):
    p = rand_problem(31, 5, 3, 2, 8, 6, 3, 0, (4,), (7,))
    for name in ("v_hist", "v_src", "v_ref"):
        setattr(p, name, np.ones_like(getattr(p, name)))
    res = O.attn(p, lib=lib)
    for kind in (TGT, SRC, REF):
        close(res[kind][0], np.ones_like(res[kind][0]), 1e-6, "V=1 gives O=1")


def _eq(a, b, what):
    assert np.array_equal(a, b), what


def pin_perturbations(lib):
    T, C = 4, 3
    p = rand_problem(41, T, C, 2, 8, cs=6, window=3, hist_first=0, ref_tokens=(3, 2),
                     ref_t0=(0, 7))
    base = O.attn(p, lib=lib)
    g = np.random.default_rng(9)
    # (1) source frame j != t: target and source rows of frame t unchanged
    for j in range(C):
        q = clone(p)
        q.k_src[j * T:(j + 1) * T] = g.standard_normal((T, 2, 8)) * 5
        q.v_src[j * T:(j + 1) * T] = g.standard_normal((T, 2, 8)) * 5
        res = O.attn(q, lib=lib)
        for t in range(C):
            sl = slice(t * T, (t + 1) * T)
            same = lambda k: (np.array_equal(res[k][0][sl], base[k][0][sl])
                              and np.array_equal(res[k][1][:, sl], base[k][1][:, sl]))
            assert same(TGT) == (t != j), "target frame %d vs perturbed source %d" % (t, j)
            assert same(SRC) == (t != j), "source frame %d vs perturbed source %d" % (t, j)
    # (2) reference image 1 (t0 = 7): frame 6 unchanged, frames 7, 8 change
    q = clone(p)
    q.k_ref[3:] = g.standard_normal((2, 2, 8)) * 5
    res = O.attn(q, lib=lib)
    _eq(res[TGT][0][:T], base[TGT][0][:T], "frame before t0 must not see image 1")
    assert not np.array_equal(res[TGT][0][T:], base[TGT][0][T:]), "frames >= t0 see image 1"
    # (3) history frames outside the window (0, 1, 2): nothing changes; frame 3 does
    q = clone(p)
    q.k_hist[:3 * T] = g.standard_normal((3 * T, 2, 8)) * 5
    res = O.attn(q, lib=lib)
    for k in (TGT, SRC, REF):
        _eq(res[k][0], base[k][0], "frames outside the window are invisible")
    q = clone(p)
    q.v_hist[3 * T:4 * T] = g.standard_normal((T, 2, 8)) * 5
    res = O.attn(q, lib=lib)
    assert not np.array_equal(res[TGT][0], base[TGT][0]), "window frame is visible"
    # (4) target tokens: source and reference rows unchanged
    q = clone(p)
    q.k_hist[:] = g.standard_normal(q.k_hist.shape) * 5
    res = O.attn(q, lib=lib)
    _eq(res[SRC][0], base[SRC][0], "source rows do not read target keys")
    _eq(res[REF][0], base[REF][0], "reference rows do not read target keys")
    # (5) source tokens: reference rows unchanged
    q = clone(p)
    q.k_src[:] = g.standard_normal(q.k_src.shape) * 5
    res = O.attn(q, lib=lib)
    _eq(res[REF][0], base[REF][0], "reference rows do not read source keys")


def pin_permutation(lib):
    T, C = 6, 3
    p = rand_problem(51, T, C, 2, 8, ref_tokens=(5,), ref_t0=(0,))
    base = O.attn(p, lib=lib)
    g = np.random.default_rng(3)
    q = clone(p)
    for f in range(C):
        perm = g.permutation(T) + f * T
        sl = slice(f * T, (f + 1) * T)
        q.k_hist[sl], q.v_hist[sl] = p.k_hist[perm], p.v_hist[perm]
        perm = g.permutation(T) + f * T
        q.k_src[sl], q.v_src[sl] = p.k_src[perm], p.v_src[perm]
    perm = g.permutation(5)
    q.k_ref, q.v_ref = p.k_ref[perm], p.v_ref[perm]
    res = O.attn(q, lib=lib)
    for k in (TGT, SRC, REF):
        close(res[k][0], base[k][0], 1e-6, "key permutation")
        close(res[k][1], base[k][1], 1e-6, "key permutation LSE")


def pin_split_merge(lib):
    # target rows with image 1 hidden (t0 huge), image 1 alone (reference rows of a problem
    # holding only image 1, queried with the target queries), merged by LSE == image 1 visible.
    T, C = 4, 2
    p = rand_problem(61, T, C, 2, 8, ref_tokens=(3, 5), ref_t0=(0, 0))
    full = O.attn(p, kinds=(TGT,), lib=lib)[TGT]
    hid = O.attn(clone(p, ref_t0=[0, 10 ** 6]), kinds=(TGT,), lib=lib)[TGT]
    img = _rows_against_keys(lib, p.q_tgt, p.k_ref[3:], p.v_ref[3:], p.D)
    lse = np.logaddexp(hid[1], img[1])
    o = (np.exp(hid[1] - lse).T[..., None] * hid[0] + np.exp(img[1] - lse).T[..., None] * img[0])
    close(o, full[0], 1e-6, "LSE merge O")
    close(lse, full[1], 1e-6, "LSE merge LSE")


def _rows_against_keys(lib, q, k, v, D):
    """Attention of arbitrary query rows against one key set, through reference rows."""
    H = q.shape[1]
    R = k.shape[0]
    outs, lses = [], []
    for i in range(q.shape[0]):
        qi = np.repeat(q[i:i + 1], R, 0)  # R reference rows, all equal to query i
        p = O.Problem(T=1, C=0, H=H, D=D, ref_tokens=[R], ref_t0=[0], q_ref=qi,
                      q_tgt=np.zeros((0, H, D), np.float32), q_src=np.zeros((0, H, D), np.float32),
                      k_hist=np.zeros((0, H, D), np.float32), v_hist=np.zeros((0, H, D), np.float32),
                      k_src=np.zeros((0, H, D), np.float32), v_src=np.zeros((0, H, D), np.float32),
                      k_ref=k, v_ref=v)
        res = O.attn(p, kinds=(REF,), lib=lib)[REF]
        outs.append(res[0][0])
        lses.append(res[1][:, 0])
    return np.stack(outs), np.stack(lses, 1)


def pin_streaming_consistency(lib):
    T, C = 5, 3
    p = rand_problem(71, T, C, 2, 8, ref_tokens=(4,), ref_t0=(1,))
    bi = O.attn(p, kinds=(TGT,), lib=lib)[TGT]
    for w in (0, 3, 12):
        st = O.attn(clone(p, window=w), kinds=(TGT,), lib=lib)[TGT]
        _eq(st[0], bi[0], "cs=0 streaming == bidirectional (window %d)" % w)
    p = rand_problem(72, T, C, 2, 8, cs=6, window=-1, ref_tokens=(4,), ref_t0=(0,))
    all_h = O.attn(p, kinds=(TGT,), lib=lib)[TGT]
    for w in (6, 7, 40):
        st = O.attn(clone(p, window=w), kinds=(TGT,), lib=lib)[TGT]
        _eq(st[0], all_h[0], "window >= cs keeps all history (window %d)" % w)
    st = O.attn(clone(p, window=5), kinds=(TGT,), lib=lib)[TGT]
    assert not np.array_equal(st[0], all_h[0]), "window < cs drops a frame"


def pin_sink(lib):
    """Sink frames (reading of the pages' sink blocks): frames 0 .. sink-1 stay visible beside
    the window.  sink = 0 is the plain window; a sink that reaches the window is all history;
    a frame neither in the sink nor in the window is invisible, a sink frame is visible."""
    T, C = 3, 2
    p = rand_problem(91, T, C, 2, 8, cs=8, window=3, hist_first=0, ref_tokens=(2,), ref_t0=(0,))
    plain = O.attn(p, kinds=(TGT,), lib=lib)[TGT]
    _eq(O.attn(clone(p, sink=0), kinds=(TGT,), lib=lib)[TGT][0], plain[0], "sink 0 = window")
    all_h = O.attn(clone(p, window=-1), kinds=(TGT,), lib=lib)[TGT]
    for sk in (5, 6, 10):  # [0, sk) u [5, 8) = all history
        st = O.attn(clone(p, sink=sk), kinds=(TGT,), lib=lib)[TGT]
        _eq(st[0], all_h[0], "sink reaching the window keeps all history (sink %d)" % sk)
    q = clone(p, sink=2)
    base = O.attn(q, kinds=(TGT,), lib=lib)[TGT]
    assert not np.array_equal(base[0], plain[0]), "sink frames are visible"
    g = np.random.default_rng(93)
    for f, visible in ((0, True), (1, True), (2, False), (4, False), (5, True)):
        r = clone(q)
        r.k_hist[f * T:(f + 1) * T] = g.standard_normal((T, 2, 8)).astype(np.float32)
        got = O.attn(r, kinds=(TGT,), lib=lib)[TGT]
        same = np.array_equal(got[0], base[0])
        assert same != visible, "frame %d visible=%s under sink 2, window 3" % (f, visible)


def pin_smoothing(lib):
    T, C = 4, 3
    p = rand_problem(81, T, C, 2, 8, cs=3, window=2, ref_tokens=(3,), ref_t0=(0,), bf16=True)
    base = O.attn(p, lib=lib)
    m = (np.random.default_rng(5).integers(-16, 16, size=(2, 8)) / 8.0).astype(np.float32)
    q = clone(p)
    for name in ("k_hist", "k_src", "k_ref"):
        setattr(q, name, getattr(p, name) - m[None])
    res = O.attn(q, lib=lib)
    for k in (TGT, SRC, REF):
        close(res[k][0], base[k][0], 2e-6, "smoothing O")
    # the LSE shifts by the (constant along a row) term scale * q.m
    shift = np.einsum("nhd,hd->hn", p.q_tgt.astype(np.float64), m.astype(np.float64)) / math.sqrt(8)
    close(res[TGT][1] + shift, base[TGT][1], 2e-6, "smoothing LSE shift")


def pin_quant_int8(lib):
    # absmax 127/128 -> scale (127/128)/127 and inverse exactly 128: codes are x*128 rounded
    # half-to-even.
    vals = np.array([127 / 128, 2.5 / 128, 3.5 / 128, -2.5 / 128, 63.5 / 128, -127 / 128,
                     0.0, 1 / 256], np.float32)
    want = np.array([127, 2, 4, -2, 64, -127, 0, 0], np.int8)
    x = np.zeros((130, 1, 8), np.float32)
    x[0, 0, :] = vals
    x[128:, 0, :] = 0.0   # second block all zero: scale 0, codes 0
    codes, scales = O.quant_int8(x, lib=lib)
    _eq(codes[0, 0], want, "hand-derived int8 codes")
    assert scales[0, 0] == np.float32(np.float32(127 / 128) / np.float32(127)), scales[0, 0]
    assert scales[0, 1] == 0 and not codes[128:].any()
    # round trip on random data with a mean: |x - m - c*s| <= s/2 and |c| reaches 127
    g = np.random.default_rng(11)
    x = g.standard_normal((300, 3, 16)).astype(np.float32) * 3
    m = g.standard_normal((3, 16)).astype(np.float32)
    codes, scales = O.quant_int8(x, mean=m, lib=lib)
    for h in range(3):
        for b in range(3):
            sl = slice(b * 128, min(300, (b + 1) * 128))
            xs = x[sl, h] - m[h]
            s = scales[h, b]
            assert abs(s - np.abs(xs).max() / 127) <= 1e-6 * s
            err = np.abs(xs - codes[sl, h].astype(np.float32) * s)
            assert err.max() <= s * 0.5 * (1 + 1e-5), (h, b, err.max() / s)
            assert np.abs(codes[sl, h]).max() == 127


def pin_quant_e4m3(lib):
    table = {0x38: 1.0, 0x7e: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0xb8: -1.0,
             0x40: 2.0, 0x3c: 1.5, 0x07: 7 * 2.0 ** -9, 0x77: 240.0}
    for c, v in table.items():
        assert O.e4m3_decode(c, lib=lib) == v, (hex(c), v)
        assert O.e4m3_encode(v, lib=lib) == c, (hex(c), v)
    assert O.e4m3_encode(1000.0, lib=lib) == 0x7e and O.e4m3_encode(-1e9, lib=lib) == 0xfe
    # ties: 1 + 1/16 lies between 1 (0x38) and 1.125 (0x39): even code wins
    assert O.e4m3_encode(1.0625, lib=lib) == 0x38
    assert O.e4m3_encode(1.1875, lib=lib) == 0x3a
    # against torch's float8_e4m3fn conversion on in-range values
    g = np.random.default_rng(12)
    xs = np.concatenate([g.standard_normal(4000) * 50, g.standard_normal(2000) * 0.01,
                         np.linspace(-448, 448, 3001)]).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(float(v), lib=lib) for v in xs], np.uint8)
    _eq(got, ref, "e4m3 encoding vs torch float8_e4m3fn")
    # block quantiser: scale = the smallest power of two 2^e with 448 * 2^e >= absmax, codes the
    # encodings of x / 2^e.  Hand-derived blocks (one head each, one block of 4 tokens):
    # absmax 448 -> scale 1 (codes are the values' own encodings); 448.5 -> 2; 1 -> 2^-8 (448/256
    # >= 1 > 448/512), the max maps to 256 (0x78); 0.875 -> 2^-9 exactly, the max maps to 448;
    # just above 0.875 -> 2^-8, the max maps to 224 (0x76); all zero -> scale 0, codes 0;
    # a subnormal absmax -> 2^-126 (the floor of e).
    cases = [(448.0, 1.0, 0x7e), (448.5, 2.0, 0x76), (1.0, 2.0 ** -8, 0x78),
             (0.875, 2.0 ** -9, 0x7e), (float(np.nextafter(np.float32(0.875), np.float32(1))),
                                         2.0 ** -8, 0x76), (0.0, 0.0, 0x00), (1e-40, 2.0 ** -126, None)]
    for amax, want_scale, want_code in cases:
        x = np.zeros((4, 1, 8), np.float32)
        x[1, 0, 3] = -amax if amax > 0 else 0.0
        x[2, 0, 0] = np.float32(amax) * np.float32(0.3)
        codes, scales = O.quant_e4m3(x, lib=lib)
        assert scales[0, 0] == np.float32(want_scale), (amax, scales[0, 0], want_scale)
        if want_code is not None:
            assert codes[1, 0, 3] == (0x80 | want_code if amax > 0 else 0), (amax, hex(codes[1, 0, 3]))
        if amax > 0:
            assert codes[2, 0, 0] == O.e4m3_encode(float(np.float32(amax) * np.float32(0.3) /
                                                         np.float32(want_scale)), lib=lib)
        assert codes[0].max() == 0 and codes[3].max() == 0
    # 448.5 / 2 = 224.25 encodes to 224 (0x76)
    x = np.zeros((1, 1, 8), np.float32)
    x[0, 0, 0] = 448.5
    assert O.quant_e4m3(x, lib=lib)[0][0, 0, 0] == 0x76
    # random blocks: power-of-two scales with 224 * s < absmax <= 448 * s, codes of x / s
    x = (g.standard_normal((300, 2, 8)) * np.array([0.01, 40.0])[None, :, None]).astype(np.float32)
    codes, scales = O.quant_e4m3(x, lib=lib)
    for h in range(2):
        for b in range(3):
            blk = x[b * 128:(b + 1) * 128, h]
            s_ = float(scales[h, b])
            am = float(np.abs(blk).max())
            assert s_ > 0 and np.frexp(s_)[0] == 0.5, s_
            assert 224 * s_ < am <= 448 * s_, (am, s_)
            want = np.array([O.e4m3_encode(float(np.float32(v) / np.float32(s_)), lib=lib)
                             for v in blk.ravel()[:64]], np.uint8)
            _eq(codes[b * 128:(b + 1) * 128, h].ravel()[:64], want, "e4m3 block codes")


def pin_kmean(lib):
    g = np.random.default_rng(13)
    segs = [g.standard_normal((n, 3, 4)).astype(np.float32) for n in (5, 9, 1)]
    m = O.kmean(segs, lib=lib)
    want = np.concatenate(segs).astype(np.float64).mean(0)
    close(m, want, 1e-7, "kmean")


def pin_w8a8_quant(lib):
    """Per-block int8 of matrices: hand-derived codes (scale absmax/127, ties to even, clamp),
    block shapes 1 x 128 and 128 x 128 with partial edges, and torch's half-to-even round."""
    x = np.zeros((2, 130), np.float32)
    x[0, :8] = [127, -63.5, 0.5, 1.5, 2.5, -2.5, 100, 0]       # absmax 127: inv 1
    x[0, 128:] = [3, -1]                                        # second block: absmax 3
    x[1, :4] = [254, 3, 5, 7]                                   # absmax 254: inv 1/2
    codes, scales = O.quant_int8_2d(x, 1, 128, lib=lib)
    assert codes[0, :8].tolist() == [127, -64, 0, 2, 2, -2, 100, 0], codes[0, :8]
    assert codes[0, 128:].tolist() == [127, -42], codes[0, 128:]  # -1 * 127/3 = -42.33
    assert codes[1, :4].tolist() == [127, 2, 2, 4], codes[1, :4]  # 1.5, 2.5, 3.5 -> 2, 2, 4
    assert scales.shape == (2, 2)
    assert scales[0, 0] == np.float32(127) / np.float32(127) and scales[1, 0] == np.float32(2)
    assert scales[0, 1] == np.float32(3) / np.float32(127) and scales[1, 1] == 0.0
    g = np.random.default_rng(5)
    w = (g.standard_normal((200, 260)) * np.exp(g.standard_normal((200, 1)))).astype(np.float32)
    for br, bc in ((1, 128), (128, 128), (64, 32)):
        codes, scales = O.quant_int8_2d(w, br, bc, lib=lib)
        for bi in range(scales.shape[0]):
            for bj in range(scales.shape[1]):
                blk = torch.from_numpy(w[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc])
                amax = blk.abs().max()
                assert scales[bi, bj] == (amax / 127).item()
                want = torch.clamp(torch.round(blk * (127 / amax)), -127, 127).to(torch.int8)
                got = codes[bi * br:(bi + 1) * br, bj * bc:(bj + 1) * bc]
                assert np.array_equal(got, want.numpy()), (br, bc, bi, bj)


def pin_w8a8_gemm(lib):
    """The W8A8 product: with unit scales it is the integer matmul (numpy int64); with scales,
    the scale-weighted sum of per-block integer matmuls; the dequantised product stays within
    the closed-form quantisation error bound of the float product."""
    g = np.random.default_rng(6)
    m, n, k = 7, 256, 384
    xq = g.integers(-127, 128, size=(m, k)).astype(np.int8)
    wq = g.integers(-127, 128, size=(n, k)).astype(np.int8)
    y = O.w8a8_gemm(xq, np.ones((m, 3), np.float32), wq, np.ones((2, 3), np.float32), lib=lib)
    assert np.array_equal(y, (xq.astype(np.int64) @ wq.astype(np.int64).T).astype(np.float64))
    sx = g.uniform(0.01, 2, size=(m, 3)).astype(np.float32)
    sw = g.uniform(0.01, 2, size=(2, 3)).astype(np.float32)
    y = O.w8a8_gemm(xq, sx, wq, sw, lib=lib)
    want = np.zeros((m, n))
    for b in range(3):
        part = xq[:, b * 128:(b + 1) * 128].astype(np.int64) @ wq[:, b * 128:(b + 1) * 128].astype(
            np.int64).T
        want += sx[:, b:b + 1].astype(np.float64) * np.repeat(sw[:, b].astype(np.float64), 128)[
            None, :] * part
    close(y, want, 1e-12, "W8A8 = scale-weighted per-block integer products")
    # quantise float matrices and compare with the float product: |x.w - xq.wq| is bounded by
    # sum_k |x||dw| + |dx||w| + |dx||dw| with |dx| <= sx/2, |dw| <= sw/2 per block
    x = g.standard_normal((m, k)).astype(np.float32)
    w = g.standard_normal((n, k)).astype(np.float32)
    xq, sx = O.quant_int8_2d(x, 1, 128, lib=lib)
    wq, sw = O.quant_int8_2d(w, 128, 128, lib=lib)
    y = O.w8a8_gemm(xq, sx, wq, sw, lib=lib)
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    dx = np.repeat(sx.astype(np.float64), 128, 1)[:, :k] / 2 * (1 + 1e-6)
    dw = np.repeat(np.repeat(sw.astype(np.float64), 128, 0)[:n], 128, 1)[:, :k] / 2 * (1 + 1e-6)
    bound = np.abs(x) @ dw.T + dx @ np.abs(w).T + dx @ dw.T
    assert np.all(np.abs(y - exact) <= bound + 1e-9)
    assert np.abs(y - exact).max() > 0  # the quantisation did something


def pin_norm_rope(lib):
    """QK-RMSNorm + three-axis RoPE (a stated reading): zero positions give the textbook RMSNorm
    (numpy), the rotation keeps each vector's norm, dot products depend only on position
    differences along every axis, and hand-derived single-pair rotations."""
    g = np.random.default_rng(8)
    N, H, D = 5, 2, 12
    x = g.standard_normal((N, H, D)).astype(np.float32)
    gamma = g.uniform(0.5, 1.5, D).astype(np.float32)
    eps = 1e-2
    z = np.zeros((N, 3), np.int32)
    out = O.norm_rope(x, gamma, eps, z, lib=lib)
    x64 = x.astype(np.float64)
    want = x64 / np.sqrt((x64 ** 2).mean(-1, keepdims=True) + eps) * gamma.astype(np.float64)
    close(out, want, 1e-6, "RoPE at position 0 is the plain RMSNorm")
    pos = g.integers(0, 50, size=(N, 3)).astype(np.int32)
    rot = O.norm_rope(x, gamma, eps, pos, lib=lib)
    close(np.linalg.norm(rot.astype(np.float64), axis=-1), np.linalg.norm(want, axis=-1), 1e-6,
          "rotation keeps the norm")
    # <rope(q, p), rope(k, p')> depends on p - p' only
    q = g.standard_normal((2, 1, 128)).astype(np.float32)
    one = np.ones(128, np.float32)
    for axis in range(3):
        dots = []
        for shift in (0, 7, 300):
            pp = np.zeros((2, 3), np.int32)
            pp[0, axis], pp[1, axis] = 11 + shift, 4 + shift
            r = O.norm_rope(q, one, 0.0, pp, lib=lib).astype(np.float64)
            dots.append(float(r[0, 0] @ r[1, 0]))
        close(dots[1:], [dots[0]] * 2, 1e-5, "relative position along axis %d" % axis)
    # D = 12: pairs (d, d+6); t pairs 0, 1; y pairs 2, 3; x pairs 4, 5; theta_j = 1e4^(-j/2)
    def single(ch, p3):
        v = np.zeros((1, 1, 12), np.float32)
        v[0, 0, ch] = 1.0
        return O.norm_rope(v, np.ones(12, np.float32), 0.0, np.array([p3], np.int32), lib=lib)[0, 0]
    r12 = np.sqrt(12.0)
    e = np.zeros(12)
    e[1], e[7] = r12 * np.cos(0.03), r12 * np.sin(0.03)    # t axis, pair j=1, t=3
    close(single(1, (3, 0, 0)), e, 1e-6, "t-axis pair")
    e = np.zeros(12)
    e[3], e[9] = r12 * np.cos(0.05), r12 * np.sin(0.05)    # y axis, pair j=1, y=5
    close(single(3, (0, 5, 0)), e, 1e-6, "y-axis pair")
    e = np.zeros(12)
    e[4], e[10] = -r12 * np.sin(2.0), r12 * np.cos(2.0)    # x axis, pair j=0 (second half), x=2
    close(single(10, (0, 0, 2)), e, 1e-6, "x-axis pair")


ALL_PINS = [pin_golden_masks, pin_bruteforce, pin_f1_full_attention, pin_two_keys,
            pin_large_scores, pin_q_zero, pin_rows_match_full,
            pin_ones_v, pin_perturbations, pin_permutation, pin_split_merge,
            pin_streaming_consistency, pin_sink, pin_smoothing, pin_quant_int8, pin_quant_e4m3, pin_kmean, pin_w8a8_quant, pin_w8a8_gemm,
            pin_norm_rope]
