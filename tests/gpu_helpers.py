"""Helpers of the GPU tests: upload seeded inputs, run libfa through its
binding, and compare with the oracle on the same (bf16-rounded) values."""
from __future__ import annotations

import math
import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

import fa_workloads as W
from frame_aligned_attention_amd import binding as B
from oracle import oracle as O

TGT, SRC, REF = O.FAO_TGT, O.FAO_SRC, O.FAO_REF
KIND_NAMES = {TGT: "tgt", SRC: "src", REF: "ref"}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype=torch.bfloat16, batch=False):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if not batch:
        t = t.unsqueeze(0)
    return t.to("cuda").to(dtype).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def lse_tol_bf16(count):
    """Diagnostic bound on |dLSE| of the bf16 kernels for a row with `count` visible keys.

    The row sum l adds the bf16-rounded p that also feed the PV product: each term carries a
    relative rounding error of at most 2^-8 (8 significant bits, nearest even), so a row
    dominated by one key can be off by up to 2^-8 ~ 3.9e-3 (the cap).  Over many keys the
    errors have random signs: their sum's relative standard deviation is about
    1.5e-3 * sqrt(sum p^2) / sum p, and for N(0,1) inputs sum p^2 / (sum p)^2 ~ e^(sigma^2) / n
    with sigma^2 ~ 1 the score variance, i.e. ~2.5e-3 / sqrt(n).  A float64 simulation of this
    arithmetic gives max |dLSE| * sqrt(n) <= 1e-2 over thousands of rows at n = 1 .. 26,520;
    0.04 / sqrt(n) is 4x that.  The 2e-5 covers fp32 accumulation, exp2 and log2.  One 64-key
    tile too many or too few moves LSE by ~64 / n: 2.4e-3 at 26,520 keys against a bound of
    2.7e-4 there; one wrong 1560-token frame moves it by ln(1 + 1560 / n) (0.057)."""
    n = np.maximum(np.asarray(count, np.float64), 1.0)
    return np.minimum(4e-3, 0.04 / np.sqrt(n) + 2e-5)


def tol_check(got, want, dtype: str, what: str, lse_got=None, lse_want=None, counts=None):
    """The contract's tolerance on O (plus an LSE diagnostic bound; `counts`, the visible-key
    count of each LSE entry, selects the bf16 bound per row).  Returns stats."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = np.abs(got - want)
    st = {"max": float(d.max()) if d.size else 0.0, "mean": float(d.mean()) if d.size else 0.0}
    if lse_got is not None:
        dl = np.abs(np.asarray(lse_got, np.float64) - np.asarray(lse_want, np.float64))
        st["lse_max"] = float(dl.max()) if dl.size else 0.0
    say("  %s: max|dO| %.3g mean|dO| %.3g max|dLSE| %.3g" % (what, st["max"], st["mean"],
                                                              st.get("lse_max", float("nan"))))
    if dtype == "f32":
        assert st["max"] <= 1e-5, (what, st)
        if "lse_max" in st:
            assert st["lse_max"] <= 1e-4, (what, st)
    elif dtype == "bf16":
        assert st["max"] <= 1e-2 and st["mean"] <= 1e-3, (what, st)
        if "lse_max" in st and dl.size:
            bound = lse_tol_bf16(np.broadcast_to(counts, dl.shape) if counts is not None
                                 else np.zeros(dl.shape))
            worst = float((dl / bound).max())
            st["lse_over_bound"] = worst
            assert worst <= 1.0, (what, st)
    else:
        g = got.ravel()
        w_ = want.ravel()
        cos = float(g @ w_ / (np.linalg.norm(g) * np.linalg.norm(w_) + 1e-30))
        st["cos"] = cos
        say("  %s: cosine %.6f" % (what, cos))
        assert cos >= 0.999 and st["max"] <= 5e-2, (what, st)
        if "lse_max" in st:  # diagnostic bound: a wrong mask moves LSE by ~0.05
            assert st["lse_max"] <= 2e-2, (what, st)
    return st


@dataclass
class Call:
    """One attention call: geometry + host fp32 inputs (bf16-exact for bf16 calls)."""
    T: int
    C: int
    H: int
    D: int
    dtype: str = "bf16"
    cs: int = 0
    window: int = 0
    cache: int = 0
    ring_first: int = -1
    ref_tokens: List[int] = field(default_factory=list)
    ref_t0: List[int] = field(default_factory=list)
    query_rows: int = 7
    q: Dict[int, np.ndarray] = field(default_factory=dict)    # kind -> [rows, H, D]
    k_hist: Optional[np.ndarray] = None  # target K of absolute frames hist_first .. cs+C-1
    v_hist: Optional[np.ndarray] = None
    hist_first: int = 0
    k_src: Optional[np.ndarray] = None
    v_src: Optional[np.ndarray] = None
    k_ref: Optional[np.ndarray] = None
    v_ref: Optional[np.ndarray] = None
    sink: int = 0  # frames 0 .. sink-1 stay visible (streaming)
    block_rows: int = 0  # bf16 work-item rows (128 or 256); 0 = the library's choice
    key_split: int = 0   # B.FA_KEY_SPLIT_AUTO or B.FA_KEY_SPLIT_OFF

    @property
    def fa_dtype(self):
        return {"f32": B.FA_F32, "bf16": B.FA_BF16, "lowbit": B.FA_LOWBIT}[self.dtype]

    def desc(self):
        return B.make_desc(self.C, self.T, self.H, self.D, ref_tokens=self.ref_tokens,
                           ref_t0=self.ref_t0, chunk_start=self.cs, window=self.window,
                           cache_frames=self.cache, query_rows=self.query_rows,
                           dtype=self.fa_dtype, sink_frames=self.sink,
                           block_rows=self.block_rows, key_split=self.key_split)

    def problem(self) -> O.Problem:
        z = np.zeros((0, self.H, self.D), np.float32)
        return O.Problem(T=self.T, C=self.C, H=self.H, D=self.D, cs=self.cs,
                         window=self.window if self.cache else -1, hist_first=self.hist_first,
                         ref_tokens=self.ref_tokens, ref_t0=self.ref_t0,
                         q_tgt=self.q.get(TGT, z), q_src=self.q.get(SRC, z), q_ref=self.q.get(REF, z),
                         k_hist=self.k_hist, v_hist=self.v_hist, k_src=self.k_src,
                         v_src=self.v_src, k_ref=self.k_ref if self.k_ref is not None else z,
                         v_ref=self.v_ref if self.v_ref is not None else z, sink=self.sink)

    def kinds(self):
        return [k for k, bit in ((TGT, 1), (SRC, 2), (REF, 4)) if self.query_rows & bit]


def random_call(seed, T, C, H, D, dtype="bf16", cs=0, window=0, cache=0, ref_tokens=(),
                ref_t0=(), query_rows=7, scale_k=1.0, sink=0, block_rows=0,
                key_split=0) -> Call:
    """Seeded N(0,1) inputs (bf16-rounded unless fp32) for one call."""
    g = np.random.default_rng(seed)

    def n(*shape):
        x = g.standard_normal(size=shape, dtype=np.float32)
        return W.round_bf16(x) if dtype != "f32" else x

    R = sum(ref_tokens)
    lo = 0 if window < 0 else max(0, cs - window)
    c = Call(T=T, C=C, H=H, D=D, dtype=dtype, cs=cs, window=window, cache=cache,
             ref_tokens=list(ref_tokens), ref_t0=list(ref_t0), query_rows=query_rows,
             hist_first=(0 if sink else lo) if cache else 0, sink=sink, block_rows=block_rows,
             key_split=key_split)
    c.q = {TGT: n(C * T, H, D), SRC: n(C * T, H, D), REF: n(R, H, D)}
    nh = (cs + C - c.hist_first) * T
    c.k_hist, c.v_hist = n(nh, H, D) * scale_k, n(nh, H, D)
    c.k_src, c.v_src = n(C * T, H, D), n(C * T, H, D)
    c.k_ref, c.v_ref = n(R, H, D), n(R, H, D)
    return c


def ring_slot(g, sink, cap):
    """The ring layout fa.h documents: sink frames keep slots 0 .. sink-1, the others cycle."""
    return g if g < sink else sink + (g - sink) % (cap - sink)


def ring_tensors(c: Call, tdtype, poison=None):
    """Ring buffers [1, cap*T, H, D] after appending frames hist_first .. cs-1 in order (each
    to its ring slot, later frames overwriting earlier ones).  Slots never written are filled
    with `poison` (None = zeros)."""
    cap, T = c.cache, c.T
    fill = 0.0 if poison is None else poison
    kr = np.full((cap * T, c.H, c.D), fill, np.float32)
    vr = np.full((cap * T, c.H, c.D), fill, np.float32)
    for g in range(c.hist_first, c.cs):
        s = ring_slot(g, c.sink, cap)
        i = (g - c.hist_first) * T
        kr[s * T:(s + 1) * T] = c.k_hist[i:i + T]
        vr[s * T:(s + 1) * T] = c.v_hist[i:i + T]
    return dev(kr, tdtype), dev(vr, tdtype)


def run_call(c: Call, poison=None, out_fill=None, layout=None, stream=None, workspace=None):
    """Runs fa_attn_fwd for the call; returns {kind: (O [rows,H,D] fp32, LSE [H,rows])}.
    workspace: a device tensor for fa_io.workspace (None: the layout's own)."""
    tdt = torch.float32 if c.dtype == "f32" else torch.bfloat16
    t = {}
    if TGT in c.kinds():
        t["q_tgt"] = dev(c.q[TGT], tdt)
    if SRC in c.kinds():
        t["q_src"] = dev(c.q[SRC], tdt)
    if REF in c.kinds() and sum(c.ref_tokens):
        t["q_ref"] = dev(c.q[REF], tdt)
    own = (c.cs - c.hist_first) * c.T
    t["k_tgt"] = dev(c.k_hist[own:], tdt)
    t["v_tgt"] = dev(c.v_hist[own:], tdt)
    t["k_src"] = dev(c.k_src, tdt)
    t["v_src"] = dev(c.v_src, tdt)
    if sum(c.ref_tokens):
        t["k_ref"] = dev(c.k_ref, tdt)
        t["v_ref"] = dev(c.v_ref, tdt)
    if c.cache:
        t["k_ring"], t["v_ring"] = ring_tensors(c, tdt, poison)
    rows = {TGT: c.C * c.T, SRC: c.C * c.T, REF: sum(c.ref_tokens)}
    outs = {}
    for k in c.kinds():
        if rows[k] == 0:
            continue
        nm = KIND_NAMES[k]
        fill = 0.0 if out_fill is None else out_fill
        t["o_" + nm] = torch.full((1, rows[k], c.H, c.D), fill, dtype=tdt, device="cuda")
        t["lse_" + nm] = torch.full((1, c.H, rows[k]), fill, dtype=torch.float32, device="cuda")
        outs[k] = nm
    L = layout or B.fa_layout_build(c.desc(), c.ring_first)
    if workspace is not None:
        t["workspace"] = workspace
    io = B.make_io(t)
    B.fa_attn_fwd(L, io, stream)
    torch.cuda.synchronize()
    return {k: (host(t["o_" + nm])[0], host(t["lse_" + nm])[0]) for k, nm in outs.items()}


def oracle_all(c: Call):
    return O.attn(c.problem(), kinds=tuple(k for k in c.kinds()
                                           if not (k == REF and sum(c.ref_tokens) == 0)))


def row_counts(p: O.Problem, kind: int, rows):
    """Visible-key count of each row from the oracle (fa_oracle_count).  The rule depends on a
    row only through its frame, so the count is taken once per frame."""
    rows = np.asarray(rows, np.int64)
    if kind == REF:
        return np.full(rows.shape, O.count(p, kind, 0) if rows.size else 0, np.int64)
    frames = rows // p.T
    per = {int(f): O.count(p, kind, int(f) * p.T) for f in np.unique(frames)}
    return np.array([per[int(f)] for f in frames], np.int64)


def compare_all(c: Call, res, what=""):
    ref = oracle_all(c)
    p = c.problem()
    stats = {}
    for k, (o, lse) in res.items():
        ro, rl = ref[k]
        cnt = row_counts(p, k, np.arange(lse.shape[1]))[None, :]  # LSE is [H, rows]
        stats[k] = tol_check(o, ro, c.dtype, "%s %s rows" % (what, KIND_NAMES[k]), lse, rl,
                             counts=cnt)
    return stats


def sample_rows(c: Call, kind: int, n: int, seed: int = 0):
    """Deterministic row sample.  Always: the first and last rows and both rows at every frame
    boundary (these are kept even when they alone exceed n).  The rest of the n rows: tile
    edges (first, middle and last row of every 128-row block), sub-sampled when there are
    more of them than room, then random rows."""
    rows = c.C * c.T if kind != REF else sum(c.ref_tokens)
    keep = {0, rows - 1}
    if kind != REF:
        for f in range(1, c.C):
            keep |= {f * c.T - 1, f * c.T}
    edges = set()
    for m in range(0, rows, 128):
        edges |= {m, min(rows - 1, m + 127), min(rows - 1, m + 63)}
    edges = sorted(edges - keep)
    g = np.random.default_rng(seed)
    room = max(0, n - len(keep))
    if len(edges) > room:
        edges = g.choice(edges, room, replace=False).tolist() if room else []
    pick = keep | set(edges)
    extra = g.integers(0, rows, size=max(0, n - len(pick)))
    return np.array(sorted(pick | set(extra.tolist())), np.int64)


def compare_sampled(c: Call, res, n_rows=96, heads=None, what=""):
    """Oracle on sampled (kind, head, row) only; the same tolerance."""
    p = c.problem()
    heads = list(range(c.H)) if heads is None else heads
    for k, (o, lse) in res.items():
        rows = sample_rows(c, k, n_rows, seed=k)
        kk, hh, rr = [], [], []
        for h in heads:
            for r in rows:
                kk.append(k); hh.append(h); rr.append(int(r))
        ro, rl = O.attn_rows(p, kk, hh, rr)
        go = np.stack([o[r, h] for h, r in zip(hh, rr)])
        gl = np.array([lse[h, r] for h, r in zip(hh, rr)])
        tol_check(go, ro, c.dtype, "%s %s rows (sampled %d)" % (what, KIND_NAMES[k], len(rr)),
                  gl, rl, counts=row_counts(p, k, rr))
