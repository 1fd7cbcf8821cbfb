"""Seeded synthetic workloads for frame-aligned attention.

Shapes of the five workloads and the seeded tensor generator that both the
tests and bench.py use.  This module holds no attention arithmetic: it only
draws numbers and names shapes.

Generator: numpy PCG64 seeded with the sequence [workload, chunk, tensor],
standard normal fp32.  For bf16 workloads the values are rounded to bf16
(round to nearest even) before anyone uses them, so a device path and the
oracle read the same numbers.

Token counts: 30x52 = 1560 and 45x80 = 3600 latent patches per frame match
480x832 and 720x1280 video at a 16-pixel latent stride (a reading: the pages
give resolutions, not token counts).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

import numpy as np

# tensor ids inside one (workload, chunk) seed
TID = {"q_tgt": 0, "k_tgt": 1, "v_tgt": 2, "q_src": 3, "k_src": 4, "v_src": 5,
       "q_ref": 6, "k_ref": 7, "v_ref": 8, "k_off": 9}


@dataclass
class Workload:
    wid: int
    name: str
    dtype: str            # "f32" | "bf16" | "lowbit"
    T: int                # tokens per frame
    C: int                # query frames per call (bidirectional: all frames)
    H: int
    D: int
    ref_tokens: List[int] = field(default_factory=list)
    ref_t0: List[int] = field(default_factory=list)   # absolute frame (relative markers below)
    ref_t0_after_cs: List[int] = field(default_factory=list)  # t0 = cs + k (-1: use ref_t0)
    window: int = 0       # target history frames; 0 for bidirectional
    cache_frames: int = 0
    chunks: int = 1       # streaming: consecutive chunks; bidirectional: 1
    first_cs: int = 0     # chunk_start of the first chunk
    query_rows: str = "tgt"   # "all" (target, source, reference rows) or "tgt"
    k_offset_var: float = 0.0  # variance of a per-(head, channel) offset added to every key

    @property
    def streaming(self) -> bool:
        return self.cache_frames > 0

    def t0_for(self, cs: int) -> List[int]:
        out = []
        for i, t0 in enumerate(self.ref_t0):
            k = self.ref_t0_after_cs[i] if i < len(self.ref_t0_after_cs) else -1
            out.append(cs + k if k >= 0 else t0)
        return out


WORKLOADS = {
    0: Workload(0, "tiny-f32", "f32", T=64, C=2, H=2, D=64, ref_tokens=[16], ref_t0=[0],
                query_rows="all"),
    1: Workload(1, "bidir-bf16-21x1560-h12", "bf16", T=1560, C=21, H=12, D=128,
                ref_tokens=[1560], ref_t0=[0], query_rows="all"),
    2: Workload(2, "stream-bf16-3x1560-w12-h40", "bf16", T=1560, C=3, H=40, D=128,
                ref_tokens=[1560], ref_t0=[0], window=12, cache_frames=12, chunks=20),
    3: Workload(3, "stream-bf16-3x3600-w9-h24-2ref", "bf16", T=3600, C=3, H=24, D=128,
                ref_tokens=[3600, 3600], ref_t0=[0, 0], ref_t0_after_cs=[-1, 1], window=9,
                cache_frames=9, chunks=1, first_cs=12),
    4: Workload(4, "stream-lowbit-3x1560-w12-h40", "lowbit", T=1560, C=3, H=40, D=128,
                ref_tokens=[1560], ref_t0=[0], window=12, cache_frames=12, chunks=20,
                k_offset_var=4.0),
}


def rng(wid: int, chunk: int, tensor: str | int) -> np.random.Generator:
    tid = TID[tensor] if isinstance(tensor, str) else int(tensor)
    return np.random.default_rng([int(wid), int(chunk), tid])


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 values."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def normal(wid: int, chunk: int, tensor: str | int, shape, bf16: bool) -> np.ndarray:
    x = rng(wid, chunk, tensor).standard_normal(size=shape, dtype=np.float32)
    return round_bf16(x) if bf16 else x


def key_offset(w: Workload) -> np.ndarray:
    """Per-(head, channel) key offset ~ N(0, var), fixed for the whole stream (fp32)."""
    if w.k_offset_var <= 0:
        return np.zeros((w.H, w.D), np.float32)
    g = rng(w.wid, 0, "k_off")
    return (g.standard_normal(size=(w.H, w.D), dtype=np.float32)
            * np.float32(np.sqrt(w.k_offset_var)))


def chunk_tensors(w: Workload, chunk: int, H: int | None = None, T: int | None = None,
                  C: int | None = None, with_queries_src_ref: bool | None = None):
    """Fresh seeded tensors of one call: q/k/v for target rows of the chunk,
    source K/V (and source queries for bidirectional workloads).  [tokens, H, D] fp32
    (bf16-rounded where the workload is bf16).  H/T/C override the workload's
    sizes for reduced test cases."""
    H = H or w.H
    T = T or w.T
    C = C or w.C
    bf = w.dtype in ("bf16", "lowbit")
    n = C * T
    out = {}
    for name in ("q_tgt", "k_tgt", "v_tgt", "k_src", "v_src"):
        out[name] = normal(w.wid, chunk, name, (n, H, w.D), bf)
    allq = w.query_rows == "all" if with_queries_src_ref is None else with_queries_src_ref
    if allq:
        out["q_src"] = normal(w.wid, chunk, "q_src", (n, H, w.D), bf)
    if w.k_offset_var > 0:
        off = key_offset(w)[:H]
        for name in ("k_tgt", "k_src"):
            out[name] = out[name] + off[None]
            if bf:
                out[name] = round_bf16(out[name])
    return out


def ref_tensors(w: Workload, H: int | None = None, ref_tokens: List[int] | None = None,
                with_queries: bool | None = None):
    """Reference-image tensors (same for the whole stream; chunk seed 0)."""
    H = H or w.H
    R = int(sum(ref_tokens if ref_tokens is not None else w.ref_tokens))
    bf = w.dtype in ("bf16", "lowbit")
    out = {}
    for name in ("k_ref", "v_ref"):
        out[name] = normal(w.wid, 0, name, (R, H, w.D), bf)
    allq = w.query_rows == "all" if with_queries is None else with_queries
    if allq:
        out["q_ref"] = normal(w.wid, 0, "q_ref", (R, H, w.D), bf)
    if w.k_offset_var > 0:
        out["k_ref"] = out["k_ref"] + key_offset(w)[:H][None]
        if bf:
            out["k_ref"] = round_bf16(out["k_ref"])
    return out


def stream_chunk_starts(w: Workload) -> List[int]:
    return [w.first_cs + i * w.C for i in range(w.chunks)]


# ---------------------------------------------------------------- per-block W8A8 linear layer

@dataclass
class LinearWorkload:
    """A linear layer y = x . w^T: x [m, k] activations, w [n, k] weights."""
    name: str
    m: int
    n: int
    k: int


# The QKV projection of one chunk of the 1560-token 40-head stream: target and source tokens of
# a 3-frame chunk (2 x 4680 rows), hidden size 40 x 128, output Q, K and V (3 x 5120).
W8A8_QKV = LinearWorkload("w8a8-qkv-9360x5120x15360", m=9360, n=15360, k=5120)


def linear_tensors(seed: int, m: int, n: int, k: int):
    """Seeded bf16-rounded activations and weights.  Activations: N(0,1) times a per-row
    log-normal scale, plus sparse large outliers (1 in 500 entries times 20), the case
    per-block scales are for; weights: N(0, 1/k)."""
    g = np.random.default_rng([1000, int(seed)])
    x = g.standard_normal((m, k), dtype=np.float32)
    x *= np.exp(0.5 * g.standard_normal((m, 1))).astype(np.float32)
    out = g.random((m, k)) < 0.002
    x[out] *= 20.0
    w = (g.standard_normal((n, k), dtype=np.float32) / np.float32(np.sqrt(k)))
    return round_bf16(x), round_bf16(w)
