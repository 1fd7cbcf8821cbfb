"""ctypes binding of libfa.so (include/fa.h).

Argument marshalling only: torch tensors (device memory) and the current torch
stream are turned into the C structures of fa.h, and every call goes to the
library.  There is no fallback: if libfa.so is missing, importing this module
raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_CAPACITY, FA_ERR_HIP, FA_ERR_NOMEM = \
    0, -1, -2, -3, -4, -5
FA_F32, FA_BF16, FA_LOWBIT = 0, 1, 2
FA_Q_TARGET, FA_Q_SOURCE, FA_Q_REF = 1, 2, 4
FA_WINDOW_ALL = -1
FA_MAX_REF = 8
FA_SEG_RING, FA_SEG_TGT, FA_SEG_SRC, FA_SEG_REF = 0, 1, 2, 3
FA_MASK_NONE, FA_MASK_SAME_FRAME, FA_MASK_GATE = 0, 1, 2
FA_QUANT_MEAN_GIVEN, FA_QUANT_RING_READY = 1, 2
FA_KEY_SPLIT_AUTO, FA_KEY_SPLIT_OFF = 0, 1


class fa_layout_desc(C.Structure):
    _fields_ = [("frames", C.c_int32), ("tokens_per_frame", C.c_int32), ("n_ref", C.c_int32),
                ("ref_tokens", C.c_int32 * FA_MAX_REF), ("ref_t0", C.c_int32 * FA_MAX_REF),
                ("chunk_start", C.c_int32), ("window", C.c_int32), ("cache_frames", C.c_int32),
                ("query_rows", C.c_int32), ("batch", C.c_int32), ("heads", C.c_int32),
                ("head_dim", C.c_int32), ("dtype", C.c_int32), ("scale", C.c_float),
                ("sink_frames", C.c_int32), ("block_rows", C.c_int32), ("key_split", C.c_int32)]


class fa_tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("stride_b", C.c_int64), ("stride_n", C.c_int64),
                ("stride_h", C.c_int64), ("scale", C.c_void_p)]


_IO_TENSORS = ["q_tgt", "q_src", "q_ref", "k_ring", "v_ring", "k_tgt", "v_tgt", "k_src", "v_src",
               "k_ref", "v_ref", "o_tgt", "o_src", "o_ref"]
_IO_PTRS = ["lse_tgt", "lse_src", "lse_ref", "k_mean", "v_absmax", "workspace"]


class fa_io(C.Structure):
    _fields_ = ([(n, fa_tensor) for n in _IO_TENSORS] + [(n, C.c_void_p) for n in _IO_PTRS] +
                [("workspace_bytes", C.c_size_t)])


class fa_tile_info(C.Structure):
    _fields_ = [("q_kind", C.c_int32), ("row0", C.c_int32), ("rows", C.c_int32),
                ("n_ranges", C.c_int32)]


class fa_range_info(C.Structure):
    _fields_ = [("seg", C.c_int32), ("begin", C.c_int32), ("end", C.c_int32), ("mask", C.c_int32),
                ("param", C.c_int32)]


def _hip_runtimes():
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return set()
    return {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libfa.so is not built (%s); run __graft_entry__.build() or "
                          "python frame_aligned_attention_amd/build.py" % LIB_PATH)
    # torch first: libfa.so must bind to the HIP runtime torch already loaded (same soname),
    # so that torch's device pointers and streams are valid in the library.
    import torch  # noqa: F401
    lib = C.CDLL(LIB_PATH)
    if len(_hip_runtimes()) > 1:
        raise ImportError("two HIP runtimes are loaded (%s); libfa.so must share torch's"
                          % sorted(_hip_runtimes()))
    P = C.c_void_p
    sig = {
        "fa_status_str": ([C.c_int], C.c_char_p),
        "fa_last_error": ([], C.c_char_p),
        "fa_layout_build": ([C.POINTER(fa_layout_desc), C.c_int32, C.POINTER(P)], C.c_int),
        "fa_layout_stats": ([P] + [C.POINTER(C.c_double)] * 4, C.c_int),
        "fa_layout_tiles": ([P] + [C.POINTER(C.c_int32)] * 3, C.c_int),
        "fa_layout_tile": ([P, C.c_int32, C.POINTER(fa_tile_info), C.POINTER(fa_range_info),
                            C.c_int32], C.c_int),
        "fa_layout_workspace_bytes": ([P, C.POINTER(C.c_size_t)], C.c_int),
        "fa_layout_splits": ([P, C.POINTER(C.c_int32), C.POINTER(C.c_int32)], C.c_int),
        "fa_layout_split": ([P, C.c_int32] + [C.POINTER(C.c_int32)] * 3 +
                            [C.c_int32, C.POINTER(fa_tile_info), C.POINTER(fa_range_info),
                             C.c_int32], C.c_int),
        "fa_layout_destroy": ([P], C.c_int),
        "fa_layout_prepare": ([P], C.c_int),
        "fa_attn_fwd": ([P, C.POINTER(fa_io), P], C.c_int),
        "fa_attn_fwd_noalloc": ([P, C.POINTER(fa_io), P], C.c_int),
        "fa_quantize_lowbit": ([P, C.POINTER(fa_io), C.POINTER(fa_io), C.c_int32, P], C.c_int),
        "fa_ring_append": ([C.POINTER(fa_layout_desc)] + [C.POINTER(fa_tensor)] * 4 +
                           [C.c_int32, C.c_int32, P], C.c_int),
        "fa_ring_quantize": ([C.POINTER(fa_layout_desc)] + [C.POINTER(fa_tensor)] * 4 +
                             [P, C.c_int32, C.c_int32, P], C.c_int),
        "fa_stream_create": ([C.POINTER(fa_layout_desc), C.POINTER(P)], C.c_int),
        "fa_stream_chunk": ([P, C.POINTER(fa_io), P], C.c_int),
        "fa_stream_advance": ([P, C.POINTER(fa_io), P], C.c_int),
        "fa_stream_layout": ([P, C.POINTER(P)], C.c_int),
        "fa_stream_state": ([P, C.POINTER(C.c_int32), C.POINTER(C.c_int32)], C.c_int),
        "fa_stream_seek": ([P, C.c_int32, C.c_int32], C.c_int),
        "fa_stream_set_refs": ([P, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32)], C.c_int),
        "fa_stream_destroy": ([P], C.c_int),
        "fa_qk_norm_rope": ([C.POINTER(fa_tensor), C.POINTER(fa_tensor), P, C.c_float, P,
                             C.c_float, C.c_int32, C.c_int32, C.c_int32, C.c_int32, P], C.c_int),
        "fa_qk_norm_rope_quant": ([C.POINTER(fa_tensor), C.POINTER(fa_tensor), P, C.c_float, P,
                                   C.c_float, C.c_int32, P, P, C.c_float, C.c_int32, C.c_int32,
                                   C.c_int32, C.c_int32, P], C.c_int),
        "fa_w8a8_quantize_act": ([P, C.c_int64, C.c_int32, C.c_int32, P, C.c_int64, P, C.c_int64,
                                  P], C.c_int),
        "fa_w8a8_quantize_weight": ([P, C.c_int64, C.c_int32, C.c_int32, P, C.c_int64, P, P],
                                    C.c_int),
        "fa_w8a8_gemm": ([P, C.c_int64, P, C.c_int64, P, C.c_int64, P, C.c_int32, C.c_int32,
                          C.c_int32, P, C.c_int64, P], C.c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.fa_last_error().decode()
        super().__init__("%s: %s (%s)" % (where, lib.fa_status_str(status).decode(), msg))


def _check(status: int, where: str):
    if status != FA_OK:
        raise FaError(status, where)


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def make_desc(frames: int, tokens_per_frame: int, heads: int, head_dim: int, *, batch: int = 1,
              ref_tokens: Sequence[int] = (), ref_t0: Sequence[int] = (), chunk_start: int = 0,
              window: int = 0, cache_frames: int = 0, query_rows: int = FA_Q_TARGET,
              dtype: int = FA_BF16, scale: float = 0.0, sink_frames: int = 0,
              block_rows: int = 0, key_split: int = FA_KEY_SPLIT_AUTO) -> fa_layout_desc:
    d = fa_layout_desc()
    d.frames, d.tokens_per_frame = frames, tokens_per_frame
    d.n_ref = len(ref_tokens)
    for i, (n, t0) in enumerate(zip(ref_tokens, ref_t0)):
        d.ref_tokens[i], d.ref_t0[i] = int(n), int(t0)
    d.chunk_start, d.window, d.cache_frames = chunk_start, window, cache_frames
    d.query_rows, d.batch, d.heads, d.head_dim = query_rows, batch, heads, head_dim
    d.dtype, d.scale = dtype, scale
    d.sink_frames = sink_frames
    d.block_rows = block_rows
    d.key_split = key_split
    return d


def tensor(t, scale=None) -> fa_tensor:
    """fa_tensor of a [B, N, H, D] or [N, H, D] torch tensor (head_dim contiguous)."""
    if t is None:
        return fa_tensor()
    if t.dim() == 3:
        sb, sn, sh = 0, t.stride(0), t.stride(1)
        dstride = t.stride(2)
    elif t.dim() == 4:
        sb, sn, sh = t.stride(0), t.stride(1), t.stride(2)
        dstride = t.stride(3)
    else:
        raise ValueError("expected a [B,N,H,D] or [N,H,D] tensor")
    if dstride != 1 and t.shape[-1] > 1:
        raise ValueError("head_dim axis must be contiguous")
    return fa_tensor(t.data_ptr(), sb, sn, sh, scale.data_ptr() if scale is not None else None)


def make_io(tensors: Dict[str, object], scales: Optional[Dict[str, object]] = None) -> fa_io:
    io = fa_io()
    scales = scales or {}
    for n in _IO_TENSORS:
        if tensors.get(n) is not None:
            setattr(io, n, tensor(tensors[n], scales.get(n)))
    for n in _IO_PTRS:
        if tensors.get(n) is not None:
            setattr(io, n, tensors[n].data_ptr())
    if tensors.get("workspace") is not None:
        ws = tensors["workspace"]
        io.workspace_bytes = ws.numel() * ws.element_size()
    return io


class Layout:
    """Owns an fa_layout*."""

    def __init__(self, handle, owned=True):
        self.handle = handle
        self.owned = owned
        self._lib = lib  # kept on the object: module globals may already be gone at exit

    def __del__(self):
        _lib = getattr(self, "_lib", None)
        if getattr(self, "owned", False) and self.handle and _lib is not None:
            _lib.fa_layout_destroy(self.handle)
            self.handle = None


def fa_layout_build(desc: fa_layout_desc, ring_first_frame: int = -1) -> Layout:
    h = C.c_void_p()
    _check(lib.fa_layout_build(C.byref(desc), ring_first_frame, C.byref(h)), "fa_layout_build")
    return Layout(h)


def fa_layout_stats(L: Layout) -> dict:
    v = [C.c_double() for _ in range(4)]
    _check(lib.fa_layout_stats(L.handle, *[C.byref(x) for x in v]), "fa_layout_stats")
    return {"useful_pairs": v[0].value, "useful_flops": v[1].value, "visited_pairs": v[2].value,
            "bytes": v[3].value}


def fa_layout_tiles(L: Layout):
    n, bm, bn = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib.fa_layout_tiles(L.handle, C.byref(n), C.byref(bm), C.byref(bn)), "fa_layout_tiles")
    return n.value, bm.value, bn.value


def fa_layout_tile(L: Layout, i: int):
    t = fa_tile_info()
    rr = (fa_range_info * 64)()
    _check(lib.fa_layout_tile(L.handle, i, C.byref(t), rr, 64), "fa_layout_tile")
    ranges = [(r.seg, r.begin, r.end, r.mask, r.param) for r in rr[:t.n_ranges]]
    return (t.q_kind, t.row0, t.rows), ranges


def fa_layout_workspace_bytes(L: Layout) -> int:
    """Bytes of key-split scratch a call with L needs (fa_io.workspace); 0 if nothing is split."""
    n = C.c_size_t()
    _check(lib.fa_layout_workspace_bytes(L.handle, C.byref(n)), "fa_layout_workspace_bytes")
    return n.value


def fa_layout_splits(L: Layout):
    """(split work items, key parts in total)."""
    n, parts = C.c_int32(), C.c_int32()
    _check(lib.fa_layout_splits(L.handle, C.byref(n), C.byref(parts)), "fa_layout_splits")
    return n.value, parts.value


def fa_layout_split(L: Layout, s: int):
    """Split item s: (tile, batch*heads + head, [(part tile, part ranges), ...])."""
    tile, bh, parts = C.c_int32(), C.c_int32(), C.c_int32()
    _check(lib.fa_layout_split(L.handle, s, C.byref(tile), C.byref(bh), C.byref(parts), -1, None,
                               None, 0), "fa_layout_split")
    out = []
    for p in range(parts.value):
        t = fa_tile_info()
        rr = (fa_range_info * 64)()
        _check(lib.fa_layout_split(L.handle, s, None, None, None, p, C.byref(t), rr, 64),
               "fa_layout_split")
        out.append(((t.q_kind, t.row0, t.rows),
                    [(r.seg, r.begin, r.end, r.mask, r.param) for r in rr[:t.n_ranges]]))
    return tile.value, bh.value, out


def fa_layout_destroy(L: Layout):
    if L.handle:
        _check(lib.fa_layout_destroy(L.handle), "fa_layout_destroy")
        L.handle = None


def fa_layout_prepare(L: Layout):
    _check(lib.fa_layout_prepare(L.handle), "fa_layout_prepare")


def fa_attn_fwd(L: Layout, io: fa_io, stream=None):
    _check(lib.fa_attn_fwd(L.handle, C.byref(io), _stream_handle(stream)), "fa_attn_fwd")


def fa_attn_fwd_noalloc(L: Layout, io: fa_io, stream=None):
    _check(lib.fa_attn_fwd_noalloc(L.handle, C.byref(io), _stream_handle(stream)),
           "fa_attn_fwd_noalloc")


def fa_quantize_lowbit(L: Layout, io_in: fa_io, io_out: fa_io, flags: int = 0, stream=None):
    _check(lib.fa_quantize_lowbit(L.handle, C.byref(io_in), C.byref(io_out), flags,
                                  _stream_handle(stream)), "fa_quantize_lowbit")


def fa_ring_append(desc: fa_layout_desc, k_ring, v_ring, k_chunk, v_chunk, first_frame: int,
                   frames: int, stream=None):
    ts = [tensor(x) for x in (k_ring, v_ring, k_chunk, v_chunk)]
    _check(lib.fa_ring_append(C.byref(desc), *[C.byref(t) for t in ts], first_frame, frames,
                              _stream_handle(stream)), "fa_ring_append")


def fa_ring_quantize(desc: fa_layout_desc, k_ring, v_ring, k_codes, v_codes, k_scales, v_scales,
                     k_mean, first_frame: int, frames: int, stream=None):
    ts = [tensor(k_ring), tensor(v_ring), tensor(k_codes, k_scales), tensor(v_codes, v_scales)]
    _check(lib.fa_ring_quantize(C.byref(desc), *[C.byref(t) for t in ts], _ptr(k_mean),
                                first_frame, frames, _stream_handle(stream)), "fa_ring_quantize")


class Stream:
    """Owns an fa_stream* (the streaming driver)."""

    def __init__(self, desc: fa_layout_desc):
        h = C.c_void_p()
        _check(lib.fa_stream_create(C.byref(desc), C.byref(h)), "fa_stream_create")
        self.handle = h
        self.desc = desc
        self._lib = lib  # kept on the object: module globals may already be gone at exit

    def __del__(self):
        _lib = getattr(self, "_lib", None)
        if getattr(self, "handle", None) and _lib is not None:
            _lib.fa_stream_destroy(self.handle)
            self.handle = None

    def chunk(self, io: fa_io, stream=None):
        _check(lib.fa_stream_chunk(self.handle, C.byref(io), _stream_handle(stream)),
               "fa_stream_chunk")

    def advance(self, io: fa_io, stream=None):
        _check(lib.fa_stream_advance(self.handle, C.byref(io), _stream_handle(stream)),
               "fa_stream_advance")

    def layout(self) -> Layout:
        h = C.c_void_p()
        _check(lib.fa_stream_layout(self.handle, C.byref(h)), "fa_stream_layout")
        return Layout(h, owned=False)

    def state(self):
        a, b = C.c_int32(), C.c_int32()
        _check(lib.fa_stream_state(self.handle, C.byref(a), C.byref(b)), "fa_stream_state")
        return a.value, b.value

    def seek(self, next_frame: int, ring_first_frame: int):
        _check(lib.fa_stream_seek(self.handle, next_frame, ring_first_frame), "fa_stream_seek")

    def set_refs(self, ref_tokens: Sequence[int], ref_t0: Sequence[int]):
        n = len(ref_tokens)
        a = (C.c_int32 * max(n, 1))(*ref_tokens)
        b = (C.c_int32 * max(n, 1))(*ref_t0)
        _check(lib.fa_stream_set_refs(self.handle, n, a, b), "fa_stream_set_refs")


def fa_stream_create(desc: fa_layout_desc) -> Stream:
    return Stream(desc)


# ---------------------------------------------------------------- per-block W8A8 linear layer

def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def fa_w8a8_quantize_act(x, xq, sx, stream=None):
    """x bf16 [m, k] (row-major, rows may be padded) -> xq int8 [m, k], sx fp32 [k/128, ld_sx]."""
    m, k = x.shape
    _check(lib.fa_w8a8_quantize_act(_ptr(x), x.stride(0), m, k, _ptr(xq), xq.stride(0), _ptr(sx),
                                    sx.stride(0), _stream_handle(stream)), "fa_w8a8_quantize_act")


def fa_w8a8_quantize_weight(w, wq, sw, stream=None):
    """w bf16 [n, k] -> wq int8 [n, k], sw fp32 [n/128, k/128]."""
    n, k = w.shape
    _check(lib.fa_w8a8_quantize_weight(_ptr(w), w.stride(0), n, k, _ptr(wq), wq.stride(0),
                                       _ptr(sw), _stream_handle(stream)), "fa_w8a8_quantize_weight")


def fa_w8a8_gemm(xq, sx, wq, sw, y, stream=None):
    """y bf16 [m, n] = W8A8 product of xq [m, k] / sx [k/128, ld_sx] and wq [n, k] / sw."""
    m, k = xq.shape
    n = wq.shape[0]
    _check(lib.fa_w8a8_gemm(_ptr(xq), xq.stride(0), _ptr(sx), sx.stride(0), _ptr(wq), wq.stride(0),
                            _ptr(sw), m, n, k, _ptr(y), y.stride(0), _stream_handle(stream)),
           "fa_w8a8_gemm")


# ---------------------------------------------------------------- QK prologue (RMSNorm + RoPE)

def fa_qk_norm_rope(x, out, gamma, pos, eps=1e-6, rope_base=10000.0, stream=None):
    """x, out bf16 [B, N, H, D] (or [N, H, D]); gamma fp32 [D]; pos int32 [N, 3]."""
    xs = x if x.dim() == 4 else x.unsqueeze(0)
    b, n, h, d = xs.shape
    ti, to = tensor(x), tensor(out)
    _check(lib.fa_qk_norm_rope(C.byref(ti), C.byref(to), _ptr(gamma), eps, _ptr(pos), rope_base,
                               n, b, h, d, _stream_handle(stream)), "fa_qk_norm_rope")


def fa_qk_norm_rope_quant(x, codes, scales, gamma, pos, is_key, k_mean=None, lse_shift=None,
                          eps=1e-6, rope_base=10000.0, softmax_scale=0.0, stream=None):
    """x bf16 [B, N, H, 128] -> codes int8 (same shape) and scales fp32 [B, H, ceil(N/128)]."""
    xs = x if x.dim() == 4 else x.unsqueeze(0)
    b, n, h, d = xs.shape
    ti, tc = tensor(x), tensor(codes, scales)
    _check(lib.fa_qk_norm_rope_quant(C.byref(ti), C.byref(tc), _ptr(gamma), eps, _ptr(pos),
                                     rope_base, int(is_key), _ptr(k_mean), _ptr(lse_shift),
                                     softmax_scale, n, b, h, d, _stream_handle(stream)),
           "fa_qk_norm_rope_quant")
