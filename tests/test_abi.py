"""libfa.so loads, exports every function include/*.h declares, and rejects bad
input on the host with the documented status codes.  No GPU needed: every
check here returns before anything is enqueued."""
import ctypes as C
import glob
import os
import re

import pytest

from frame_aligned_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fa_layout_build", "fa_layout_stats", "fa_layout_destroy", "fa_attn_fwd",
              "fa_quantize_lowbit", "fa_ring_append", "fa_status_str", "fa_last_error",
              "fa_stream_create", "fa_stream_chunk", "fa_stream_advance", "fa_stream_state",
              "fa_stream_seek", "fa_stream_set_refs", "fa_stream_layout", "fa_stream_destroy",
              "fa_layout_tiles", "fa_layout_tile"):
        assert n in names, n


@pytest.mark.parametrize("name", declared_functions())
def test_symbol_exported(name):
    lib = C.CDLL(B.LIB_PATH)
    assert hasattr(lib, name), name


def test_status_strings():
    for s, t in [(0, "FA_OK"), (-1, "FA_ERR_INVALID"), (-2, "FA_ERR_UNSUPPORTED"),
                 (-3, "FA_ERR_CAPACITY"), (-4, "FA_ERR_HIP"), (-5, "FA_ERR_NOMEM")]:
        assert B.lib.fa_status_str(s).decode() == t


def desc(**kw):
    base = dict(frames=3, tokens_per_frame=40, heads=2, head_dim=128, ref_tokens=[16],
                ref_t0=[0], chunk_start=6, window=3, cache_frames=4, dtype=B.FA_BF16)
    base.update(kw)
    args = {k: base.pop(k) for k in ("frames", "tokens_per_frame", "heads", "head_dim")}
    return B.make_desc(args["frames"], args["tokens_per_frame"], args["heads"], args["head_dim"],
                       **base)


def build_status(d, ring_first=-1):
    h = C.c_void_p()
    st = B.lib.fa_layout_build(C.byref(d), ring_first, C.byref(h))
    if st == 0:
        B.lib.fa_layout_destroy(h)
    return st


@pytest.mark.parametrize("kw,status", [
    (dict(frames=0), B.FA_ERR_INVALID),
    (dict(tokens_per_frame=0), B.FA_ERR_INVALID),
    (dict(head_dim=96), B.FA_ERR_UNSUPPORTED),
    (dict(heads=0), B.FA_ERR_INVALID),
    (dict(batch=0), B.FA_ERR_INVALID),
    (dict(window=-2), B.FA_ERR_INVALID),
    (dict(chunk_start=-1), B.FA_ERR_INVALID),
    (dict(cache_frames=-1), B.FA_ERR_INVALID),
    (dict(query_rows=0), B.FA_ERR_INVALID),
    (dict(query_rows=8), B.FA_ERR_INVALID),
    (dict(dtype=7), B.FA_ERR_INVALID),
    (dict(dtype=B.FA_LOWBIT, head_dim=64), B.FA_ERR_UNSUPPORTED),
    (dict(scale=-1.0), B.FA_ERR_INVALID),
    (dict(scale=float("nan")), B.FA_ERR_INVALID),
    (dict(window=3, cache_frames=2), B.FA_ERR_CAPACITY),        # ring smaller than window
    (dict(window=-1, cache_frames=4), B.FA_ERR_CAPACITY),       # all history, 6 frames > 4
    (dict(tokens_per_frame=1 << 29, frames=2), B.FA_ERR_UNSUPPORTED),
    (dict(sink_frames=-1), B.FA_ERR_INVALID),
    (dict(sink_frames=2, cache_frames=5), B.FA_OK),              # 2 sink slots + 3 for the window
    (dict(sink_frames=2, cache_frames=4), B.FA_ERR_CAPACITY),    # 2 cycling slots < window 3
    (dict(sink_frames=5, window=0, cache_frames=4), B.FA_ERR_CAPACITY),  # 5 sink frames, 4 slots
    (dict(sink_frames=6, window=0, cache_frames=6), B.FA_OK),    # history = the 6 sink frames
    (dict(sink_frames=4, window=3, cache_frames=6), B.FA_OK),    # sink reaches the window
    (dict(block_rows=128), B.FA_OK),
    (dict(block_rows=256), B.FA_OK),
    (dict(block_rows=192), B.FA_ERR_INVALID),
    (dict(block_rows=512), B.FA_ERR_INVALID),
    (dict(block_rows=128, dtype=B.FA_LOWBIT), B.FA_ERR_INVALID),  # bf16 only
    (dict(block_rows=128, dtype=B.FA_F32), B.FA_ERR_INVALID),
    (dict(), B.FA_OK),
    (dict(window=0, cache_frames=0), B.FA_OK),
    (dict(chunk_start=0, window=-1, cache_frames=0), B.FA_OK),  # no history at all
])
def test_descriptor_validation(kw, status):
    assert build_status(desc(**kw)) == status, B.lib.fa_last_error().decode()


def test_too_many_refs_and_negative_ref_tokens():
    d = desc()
    d.n_ref = 9
    assert build_status(d) == B.FA_ERR_INVALID
    d = desc()
    d.ref_tokens[0] = -1
    assert build_status(d) == B.FA_ERR_INVALID


def test_ring_first_frame_checks():
    d = desc()  # cs 6, window 3 -> history frames 3, 4, 5
    assert build_status(d, 3) == B.FA_OK
    assert build_status(d, 2) == B.FA_OK          # ring holds 2..5 (capacity 4)
    assert build_status(d, 4) == B.FA_ERR_CAPACITY  # frame 3 missing
    assert build_status(d, 1) == B.FA_ERR_INVALID   # 1..5 is 5 frames > capacity 4
    assert build_status(d, 7) == B.FA_ERR_INVALID   # after chunk_start


def test_ring_first_frame_checks_with_sink():
    d = desc(sink_frames=1, cache_frames=5)  # cs 6, window 3: sink 0 + frames 3, 4, 5
    assert build_status(d, 3) == B.FA_OK
    assert build_status(d, 2) == B.FA_OK          # cycling slots hold 2..5 (4 slots)
    assert build_status(d, 4) == B.FA_ERR_CAPACITY  # frame 3 missing
    assert build_status(d, 1) == B.FA_ERR_INVALID   # 1..5 is 5 frames > 4 cycling slots


def test_last_error_is_set():
    build_status(desc(head_dim=96))
    assert "head_dim" in B.lib.fa_last_error().decode()


def test_attn_fwd_rejects_bad_io_on_host():
    L = B.fa_layout_build(desc())
    io = B.fa_io()
    st = B.lib.fa_attn_fwd(L.handle, C.byref(io), None)
    assert st == B.FA_ERR_INVALID and "NULL" in B.lib.fa_last_error().decode()
    # a misaligned base pointer is rejected before any launch
    io = B.fa_io()
    for n in B._IO_TENSORS:
        getattr(io, n).data = 0x1000
        getattr(io, n).stride_n = 256
        getattr(io, n).stride_h = 128
    io.q_tgt.data = 0x1002
    st = B.lib.fa_attn_fwd(L.handle, C.byref(io), None)
    assert st == B.FA_ERR_INVALID and "aligned" in B.lib.fa_last_error().decode()
    io.q_tgt.data = 0x1000
    io.k_src.stride_n = 100  # 200 bytes: rows not 16-byte aligned
    st = B.lib.fa_attn_fwd(L.handle, C.byref(io), None)
    assert st == B.FA_ERR_INVALID
    st = B.lib.fa_attn_fwd(None, C.byref(io), None)
    assert st == B.FA_ERR_INVALID


def test_ring_append_rejects_bad_args_on_host():
    d = desc()
    t = B.fa_tensor(0x1000, 0, 256, 128, None)
    assert B.lib.fa_ring_append(C.byref(d), C.byref(t), C.byref(t), C.byref(t), C.byref(t), 0, 5,
                                None) == B.FA_ERR_INVALID  # more frames than capacity
    assert B.lib.fa_ring_append(C.byref(d), C.byref(t), C.byref(t), C.byref(t), C.byref(t), -1, 1,
                                None) == B.FA_ERR_INVALID
    bad = B.fa_tensor(0x1001, 0, 256, 128, None)
    assert B.lib.fa_ring_append(C.byref(d), C.byref(bad), C.byref(t), C.byref(t), C.byref(t), 0,
                                1, None) == B.FA_ERR_INVALID
    assert B.lib.fa_ring_append(C.byref(d), C.byref(t), C.byref(t), C.byref(t), C.byref(t), 0, 0,
                                None) == B.FA_OK  # nothing to do
    d = desc(sink_frames=2)  # 2 sink slots, 2 cycling slots
    assert B.lib.fa_ring_append(C.byref(d), C.byref(t), C.byref(t), C.byref(t), C.byref(t), 4, 3,
                                None) == B.FA_ERR_INVALID  # 3 non-sink frames > 2 cycling slots
    d = desc(sink_frames=5)  # more sink frames than slots
    assert B.lib.fa_ring_append(C.byref(d), C.byref(t), C.byref(t), C.byref(t), C.byref(t), 0, 0,
                                None) == B.FA_ERR_INVALID
    d = desc(batch=40000)  # the launch grid holds tensor and batch in its y dimension
    assert B.lib.fa_ring_append(C.byref(d), C.byref(t), C.byref(t), C.byref(t), C.byref(t), 0, 1,
                                None) == B.FA_ERR_UNSUPPORTED


def test_stream_state_and_seek():
    d = desc(chunk_start=0, window=12, cache_frames=12)
    s = B.Stream(d)
    assert s.state() == (0, 0)
    s.seek(12, 3)
    assert s.state() == (12, 3)
    with pytest.raises(B.FaError):
        s.seek(12, 13)
    with pytest.raises(B.FaError):
        s.seek(30, 3)  # 27 frames cannot be in a 12-frame ring
    s2 = B.Stream(desc(chunk_start=0, window=4, cache_frames=7, sink_frames=2))
    s2.seek(20, 15)  # sink 0, 1 and frames 15..19 in the 5 cycling slots
    assert s2.state() == (20, 15)
    with pytest.raises(B.FaError):
        s2.seek(20, 14)  # 6 non-sink frames > 5 cycling slots
    s.set_refs([16, 8], [0, 14])
    with pytest.raises(B.FaError):
        s.set_refs([1] * 9, [0] * 9)


def test_w8a8_gemm_argument_checks():
    """fa_w8a8_gemm rejects bad shapes, alignment and leading dimensions on the host (every case
    returns before a launch; the pointers are aligned stand-ins that are never dereferenced)."""
    P = C.c_void_p
    ptr = 0x10000
    base = dict(xq=ptr, ld_xq=256, sx=ptr, ld_sx=64, wq=ptr, ld_wq=256, sw=ptr, m=64, n=128,
                k=256, y=ptr, ld_y=128)

    def call(**kw):
        a = {**base, **kw}
        return B.lib.fa_w8a8_gemm(P(a["xq"]), a["ld_xq"], P(a["sx"]), a["ld_sx"], P(a["wq"]),
                                  a["ld_wq"], P(a["sw"]), a["m"], a["n"], a["k"], P(a["y"]),
                                  a["ld_y"], None)

    assert call(m=0) == B.FA_OK and call(n=0) == B.FA_OK  # nothing to do
    for kw in (dict(n=100), dict(k=200), dict(k=0), dict(m=-1), dict(ld_xq=255),
               dict(ld_xq=264), dict(ld_wq=200), dict(ld_y=120), dict(ld_sx=63),
               dict(xq=ptr + 8), dict(y=ptr + 4), dict(sx=ptr + 2), dict(xq=0)):
        assert call(**kw) == B.FA_ERR_INVALID, kw
    # a 256-row activation tile must stay within 32-bit offsets
    assert call(ld_xq=1 << 23, k=256) == B.FA_ERR_UNSUPPORTED
    assert call(ld_y=1 << 22, n=128) == B.FA_ERR_UNSUPPORTED  # 2^23 bytes of bf16


def test_per_source_build_flags():
    """A source's `// build-flags:` line is what the build passes for it (and it sits in the
    hashed source text); only the two attention files with row maxima ask for any (no NaN
    quieting before the maxima)."""
    from frame_aligned_attention_amd import build as fb
    flags = {os.path.basename(s): fb.file_flags(s) for s in fb.sources()}
    with_flags = ("fa_attn_bf16.hip", "fa_lowbit.hip")
    for k in with_flags:
        assert flags[k] == ["-fno-honor-nans"], k
    assert all(v == [] for k, v in flags.items() if k not in with_flags)
