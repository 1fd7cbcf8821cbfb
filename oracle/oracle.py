"""ctypes binding of the CPU oracle (oracle/fa_oracle.c).

Test infrastructure only.  `build()` compiles liboracle.so with gcc and
OpenMP; the functions below marshal numpy arrays (fp32, token-major
[tokens, H, D]) and call the C code.  No arithmetic of the method lives here.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

FAO_TGT, FAO_SRC, FAO_REF = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_HDR = os.path.join(_HERE, "fa_oracle.h")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False, out: Optional[str] = None, src: Optional[str] = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Returns the library path.

    `src`/`out` let a test compile a modified copy elsewhere; by default the
    in-tree source is built next to it, and only when it is newer than the
    library (or `force`)."""
    src = src or _SRC
    out = out or _LIB
    if not force and os.path.exists(out) and src == _SRC:
        if os.path.getmtime(out) >= max(os.path.getmtime(_SRC), os.path.getmtime(_HDR)):
            return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-I", os.path.dirname(os.path.abspath(src)),
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(path: str):
    lib = C.CDLL(path)
    fp = C.POINTER(C.c_float)
    ip = C.POINTER(C.c_int)
    lib.fa_oracle_attn.argtypes = [C.c_void_p, C.c_int] + [fp] * 6
    lib.fa_oracle_attn.restype = C.c_int
    lib.fa_oracle_attn_rows.argtypes = [C.c_void_p, C.c_int, ip, ip, ip, fp, fp]
    lib.fa_oracle_attn_rows.restype = C.c_int
    lib.fa_oracle_count.argtypes = [C.c_void_p, C.c_int, C.c_int]
    lib.fa_oracle_count.restype = C.c_long
    lib.fa_oracle_threads.restype = C.c_int
    lib.fa_oracle_quant_int8.argtypes = [fp, C.c_int, C.c_int, C.c_int, fp,
                                         C.POINTER(C.c_int8), fp]
    lib.fa_oracle_quant_e4m3.argtypes = [fp, C.c_int, C.c_int, C.c_int, fp,
                                         C.POINTER(C.c_uint8), fp]
    lib.fa_oracle_e4m3_encode.argtypes = [C.c_float]
    lib.fa_oracle_e4m3_encode.restype = C.c_uint8
    lib.fa_oracle_e4m3_decode.argtypes = [C.c_uint8]
    lib.fa_oracle_e4m3_decode.restype = C.c_float
    lib.fa_oracle_kmean.argtypes = [C.c_int, C.POINTER(fp), ip, C.c_int, C.c_int, fp]
    lib.fa_oracle_quant_int8_2d.argtypes = [fp, C.c_int, C.c_int, C.c_int, C.c_int,
                                            C.POINTER(C.c_int8), fp]
    i8p = C.POINTER(C.c_int8)
    lib.fa_oracle_w8a8_gemm.argtypes = [i8p, fp, i8p, fp, C.c_int, C.c_int, C.c_int,
                                        C.POINTER(C.c_double)]
    lib.fa_oracle_norm_rope.argtypes = [fp, C.c_int, C.c_int, C.c_int, fp, C.c_double, ip,
                                        C.c_double, fp]
    return lib


def load(path: Optional[str] = None):
    """The oracle library (built on first use).  `path` loads another build."""
    global _lib
    if path is not None:
        return _bind(path)
    if _lib is None:
        _lib = _bind(build())
    return _lib


class _CProblem(C.Structure):
    _fields_ = [
        ("T", C.c_int), ("C", C.c_int), ("cs", C.c_int), ("window", C.c_int),
        ("hist_first", C.c_int), ("n_ref", C.c_int),
        ("ref_tokens", C.POINTER(C.c_int)), ("ref_t0", C.POINTER(C.c_int)),
        ("H", C.c_int), ("D", C.c_int), ("scale", C.c_double),
        ("q_tgt", C.c_void_p), ("q_src", C.c_void_p), ("q_ref", C.c_void_p),
        ("k_hist", C.c_void_p), ("v_hist", C.c_void_p),
        ("k_src", C.c_void_p), ("v_src", C.c_void_p),
        ("k_ref", C.c_void_p), ("v_ref", C.c_void_p),
        ("sink", C.c_int),
    ]


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


@dataclass
class Problem:
    """One call's worth of inputs.  Arrays are [tokens, H, D] fp32.

    k_hist / v_hist hold target frames hist_first .. cs+C-1 by absolute frame
    (the current chunk's own target K/V are its last C frames).  sink: frames
    0 .. sink-1 stay visible to target rows beside the window (streaming)."""
    T: int
    C: int
    H: int
    D: int
    cs: int = 0
    window: int = -1
    hist_first: int = 0
    ref_tokens: Sequence[int] = ()
    ref_t0: Sequence[int] = ()
    scale: Optional[float] = None
    q_tgt: Optional[np.ndarray] = None
    q_src: Optional[np.ndarray] = None
    q_ref: Optional[np.ndarray] = None
    k_hist: Optional[np.ndarray] = None
    v_hist: Optional[np.ndarray] = None
    k_src: Optional[np.ndarray] = None
    v_src: Optional[np.ndarray] = None
    k_ref: Optional[np.ndarray] = None
    v_ref: Optional[np.ndarray] = None
    sink: int = 0
    _keep: list = field(default_factory=list, repr=False)

    def rows(self, kind: int) -> int:
        return int(sum(self.ref_tokens)) if kind == FAO_REF else self.C * self.T

    def _c(self):
        n = len(self.ref_tokens)
        rt = (C.c_int * max(n, 1))(*[int(x) for x in self.ref_tokens])
        r0 = (C.c_int * max(n, 1))(*[int(x) for x in self.ref_t0])
        scale = self.scale if self.scale is not None else 1.0 / np.sqrt(self.D)
        keep = [rt, r0]
        arrs = {}
        for name in ("q_tgt", "q_src", "q_ref", "k_hist", "v_hist", "k_src", "v_src",
                     "k_ref", "v_ref"):
            a = _f32(getattr(self, name))
            keep.append(a)
            arrs[name] = a.ctypes.data if a is not None and a.size else None
        self._keep = keep
        return _CProblem(self.T, self.C, self.cs, self.window, self.hist_first, n, rt, r0,
                         self.H, self.D, float(scale), **arrs, sink=int(self.sink))


def _fp(a):
    return a.ctypes.data_as(C.POINTER(C.c_float)) if a is not None else None


def attn(p: Problem, kinds=(FAO_TGT, FAO_SRC, FAO_REF), lib=None):
    """All rows of the given query kinds.  Returns {kind: (o [rows,H,D], lse [H,rows])}."""
    lib = lib or load()
    cp = p._c()
    outs = {}
    ptrs = []
    mask = 0
    for kind in (FAO_TGT, FAO_SRC, FAO_REF):
        if kind in kinds:
            rows = p.rows(kind)
            o = np.zeros((rows, p.H, p.D), np.float32)
            lse = np.zeros((p.H, rows), np.float32)
            outs[kind] = (o, lse)
            mask |= 1 << kind
            ptrs += [_fp(o), _fp(lse)]
        else:
            ptrs += [None, None]
    rc = lib.fa_oracle_attn(C.byref(cp), mask, *ptrs)
    if rc != 0:
        raise ValueError("oracle rejected the problem (code %d)" % rc)
    return outs


def attn_rows(p: Problem, kind, head, row, lib=None):
    """Selected rows: arrays kind/head/row of equal length -> (o [n,D], lse [n])."""
    lib = lib or load()
    cp = p._c()
    kind = np.ascontiguousarray(kind, dtype=np.int32)
    head = np.ascontiguousarray(head, dtype=np.int32)
    row = np.ascontiguousarray(row, dtype=np.int32)
    n = len(kind)
    o = np.zeros((n, p.D), np.float32)
    lse = np.zeros((n,), np.float32)
    ip = C.POINTER(C.c_int)
    rc = lib.fa_oracle_attn_rows(C.byref(cp), n, kind.ctypes.data_as(ip),
                                 head.ctypes.data_as(ip), row.ctypes.data_as(ip), _fp(o), _fp(lse))
    if rc != 0:
        raise ValueError("oracle rejected the rows (code %d)" % rc)
    return o, lse


def count(p: Problem, kind: int, row: int, lib=None) -> int:
    lib = lib or load()
    cp = p._c()
    return int(lib.fa_oracle_count(C.byref(cp), kind, row))


def threads(lib=None) -> int:
    return int((lib or load()).fa_oracle_threads())


def quant_int8(x, mean=None, lib=None):
    """x [N,H,D] fp32 -> (codes int8 [N,H,D], scales [H, ceil(N/128)])."""
    lib = lib or load()
    x = _f32(x)
    N, H, D = x.shape
    codes = np.zeros(x.shape, np.int8)
    scales = np.zeros((H, (N + 127) // 128), np.float32)
    m = _f32(mean)
    lib.fa_oracle_quant_int8(_fp(x), N, H, D, _fp(m), codes.ctypes.data_as(C.POINTER(C.c_int8)),
                             _fp(scales))
    return codes, scales


def quant_e4m3(x, mean=None, lib=None):
    """x [N,H,D] fp32 -> (codes uint8 e4m3 [N,H,D], scales [H, ceil(N/128)])."""
    lib = lib or load()
    x = _f32(x)
    N, H, D = x.shape
    codes = np.zeros(x.shape, np.uint8)
    scales = np.zeros((H, (N + 127) // 128), np.float32)
    m = _f32(mean)
    lib.fa_oracle_quant_e4m3(_fp(x), N, H, D, _fp(m),
                             codes.ctypes.data_as(C.POINTER(C.c_uint8)), _fp(scales))
    return codes, scales


def e4m3_encode(x: float, lib=None) -> int:
    return int((lib or load()).fa_oracle_e4m3_encode(float(x)))


def e4m3_decode(c: int, lib=None) -> float:
    return float((lib or load()).fa_oracle_e4m3_decode(int(c)))


def kmean(segs, lib=None):
    """Per-head, per-channel mean over the rows of several [n,H,D] arrays -> [H,D]."""
    lib = lib or load()
    segs = [_f32(s) for s in segs]
    H, D = segs[0].shape[1:]
    fp = C.POINTER(C.c_float)
    arr = (fp * len(segs))(*[_fp(s) for s in segs])
    ntok = (C.c_int * len(segs))(*[s.shape[0] for s in segs])
    mean = np.zeros((H, D), np.float32)
    lib.fa_oracle_kmean(len(segs), arr, ntok, H, D, _fp(mean))
    return mean


def quant_int8_2d(x, br, bc, lib=None):
    """Per-block int8 of a [rows, cols] matrix in br x bc blocks -> (codes int8 [rows, cols],
    scales [ceil(rows/br), ceil(cols/bc)])."""
    lib = lib or load()
    x = _f32(x)
    rows, cols = x.shape
    codes = np.zeros(x.shape, np.int8)
    scales = np.zeros(((rows + br - 1) // br, (cols + bc - 1) // bc), np.float32)
    lib.fa_oracle_quant_int8_2d(_fp(x), rows, cols, br, bc,
                                codes.ctypes.data_as(C.POINTER(C.c_int8)), _fp(scales))
    return codes, scales


def w8a8_gemm(xq, sx, wq, sw, lib=None):
    """Per-block W8A8 product: xq [m,k] int8, sx [m, ceil(k/128)], wq [n,k] int8,
    sw [ceil(n/128), ceil(k/128)] -> y [m,n] float64."""
    lib = lib or load()
    xq = np.ascontiguousarray(xq, np.int8)
    wq = np.ascontiguousarray(wq, np.int8)
    sx, sw = _f32(sx), _f32(sw)
    m, k = xq.shape
    n = wq.shape[0]
    y = np.zeros((m, n), np.float64)
    i8p = C.POINTER(C.c_int8)
    lib.fa_oracle_w8a8_gemm(xq.ctypes.data_as(i8p), _fp(sx), wq.ctypes.data_as(i8p), _fp(sw),
                            m, n, k, y.ctypes.data_as(C.POINTER(C.c_double)))
    return y


def norm_rope(x, gamma, eps, pos, base=10000.0, lib=None):
    """QK-RMSNorm + three-axis RoPE: x [N,H,D] fp32, gamma [D], pos [N,3] int -> [N,H,D]."""
    lib = lib or load()
    x = _f32(x)
    N, H, D = x.shape
    assert D <= 1024 and D % 2 == 0
    g = _f32(gamma)
    p = np.ascontiguousarray(pos, np.int32)
    out = np.zeros_like(x)
    lib.fa_oracle_norm_rope(_fp(x), N, H, D, _fp(g), float(eps),
                            p.ctypes.data_as(C.POINTER(C.c_int)), float(base), _fp(out))
    return out
