"""Per-block W8A8 linear layer on the GPU against the oracle: quantiser codes and scales
bit-exact; the GEMM within the tolerance its arithmetic allows (exact int32 block products, fp32
dequantised accumulation, one bf16 rounding):
  |y - y_ref| <= 2^-8 |y_ref| + (k/128 + 4) 2^-23 S,
with S the sum over blocks of |sx sw dot| (the oracle's product of the absolute codes)."""
import numpy as np
import pytest
import torch

import fa_workloads as W
import gpu_helpers as G
from frame_aligned_attention_amd import binding as B
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def quantise_on_gpu(x, w, pad=0):
    """Device quantisation of x [m,k] and w [n,k] (host fp32, bf16-exact); returns device codes
    and scales (sx as [k/128, ld_sx]).  `pad` widens every leading dimension."""
    m, k = x.shape
    n = w.shape[0]
    xd = torch.zeros((m, k + pad), dtype=torch.bfloat16, device="cuda")[:, :k]
    xd.copy_(torch.from_numpy(x))
    wd = torch.zeros((n, k + pad), dtype=torch.bfloat16, device="cuda")[:, :k]
    wd.copy_(torch.from_numpy(w))
    xq = torch.zeros((m, k + pad), dtype=torch.int8, device="cuda")[:, :k]
    wq = torch.zeros((n, k + pad), dtype=torch.int8, device="cuda")[:, :k]
    sx = torch.zeros((k // 128, m + pad), dtype=torch.float32, device="cuda")
    sw = torch.zeros((n // 128, k // 128), dtype=torch.float32, device="cuda")
    B.fa_w8a8_quantize_act(xd, xq, sx)
    B.fa_w8a8_quantize_weight(wd, wq, sw)
    torch.cuda.synchronize()
    return xq, sx, wq, sw


def check_codes(x, w, xq, sx, wq, sw):
    m, k = x.shape
    cx, scx = O.quant_int8_2d(x, 1, 128)
    cw, scw = O.quant_int8_2d(w, 128, 128)
    assert np.array_equal(xq.cpu().numpy(), cx)
    assert np.array_equal(sx.cpu().numpy()[:, :m].T, scx)
    assert np.array_equal(wq.cpu().numpy(), cw)
    assert np.array_equal(sw.cpu().numpy(), scw)
    return cx, scx, cw, scw


def check_gemm(y, cx, scx, cw, scw, rows=None, what=""):
    """y: host fp32 of the device output (rows `rows` of the full product, or all)."""
    if rows is not None:
        cx, scx = cx[rows], scx[rows]
    ref = O.w8a8_gemm(cx, scx, cw, scw)
    S = O.w8a8_gemm(np.abs(cx.astype(np.int16)).astype(np.int8), scx,
                    np.abs(cw.astype(np.int16)).astype(np.int8), scw)
    kbt = cx.shape[1] // 128
    tol = 2.0 ** -8 * np.abs(ref) + (kbt + 4) * 2.0 ** -23 * S
    err = np.abs(y.astype(np.float64) - ref)
    G.say("  %s: max|dy| %.3g, max|dy|/tol %.3f, max|y| %.3g" % (what, err.max(),
                                                                 (err / tol).max(), np.abs(ref).max()))
    assert np.all(err <= tol), what


CASES = [  # m, n, k, leading-dimension padding
    (1, 128, 128, 0),
    (37, 256, 384, 0),
    (130, 128, 256, 16),   # ragged m across two tiles, padded rows
    (300, 384, 640, 0),
    (257, 128, 1024, 32),
    (513, 1024, 768, 0),    # 8 n tiles (the XCD-grouped order), 6 K-blocks: one unrolled loop pass
    (600, 1152, 1664, 16),  # 9 n tiles split unevenly over the XCDs, 13 K-blocks
]


@pytest.mark.parametrize("case", CASES, ids=["m%d_n%d_k%d" % c[:3] for c in CASES])
def test_w8a8_quantisers_and_gemm(case):
    m, n, k, pad = case
    G.say("case: W8A8 m=%d n=%d k=%d pad=%d" % case)
    x, w = W.linear_tensors(m * 7 + n + k, m, n, k)
    xq, sx, wq, sw = quantise_on_gpu(x, w, pad)
    cx, scx, cw, scw = check_codes(x, w, xq, sx, wq, sw)
    y = torch.full((m, n + pad), float("nan"), dtype=torch.bfloat16, device="cuda")[:, :n]
    B.fa_w8a8_gemm(xq, sx, wq, sw, y)
    torch.cuda.synchronize()
    check_gemm(y.float().cpu().numpy(), cx, scx, cw, scw, what="gemm")
    if pad:  # nothing written outside [m, n]
        full = y.as_strided((m, n + pad), (y.stride(0), 1))
        assert torch.isnan(full[:, n:].float()).all()


def test_w8a8_unit_scales_integer_product():
    G.say("case: W8A8 GEMM with unit scales equals the integer product")
    g = np.random.default_rng(3)
    m, n, k = 64, 128, 256
    cx = g.integers(-127, 128, size=(m, k)).astype(np.int8)
    cw = g.integers(-127, 128, size=(n, k)).astype(np.int8)
    xq = torch.from_numpy(cx).cuda()
    wq = torch.from_numpy(cw).cuda()
    sx = torch.ones((k // 128, m), dtype=torch.float32, device="cuda")
    sw = torch.ones((n // 128, k // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    B.fa_w8a8_gemm(xq, sx, wq, sw, y)
    torch.cuda.synchronize()
    exact = torch.from_numpy(cx.astype(np.int64) @ cw.astype(np.int64).T).double()
    assert torch.equal(y.double().cpu(), exact.to(torch.bfloat16).double())


def test_w8a8_qkv_projection_full_size_sampled():
    wl = W.W8A8_QKV
    G.say("case: %s full size, sampled rows" % wl.name)
    x, w = W.linear_tensors(1, wl.m, wl.n, wl.k)
    xq, sx, wq, sw = quantise_on_gpu(x, w)
    y = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device="cuda")
    B.fa_w8a8_gemm(xq, sx, wq, sw, y)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 4679, 4680, wl.m - 129, wl.m - 1} |
                           set(np.random.default_rng(0).integers(0, wl.m, 8).tolist())))
    cx = xq.cpu().numpy()
    scx = sx.cpu().numpy().T
    # the sampled rows' codes and scales against the oracle quantiser, then the product
    ocx, oscx = O.quant_int8_2d(x[rows], 1, 128)
    assert np.array_equal(cx[rows], ocx) and np.array_equal(scx[rows], oscx)
    cw, scw = O.quant_int8_2d(w, 128, 128)
    assert np.array_equal(wq.cpu().numpy(), cw) and np.array_equal(sw.cpu().numpy(), scw)
    check_gemm(y.float().cpu().numpy()[rows], cx, scx, cw, scw, rows=rows, what="sampled rows")
    # and the dequantised product tracks the float product (quantisation error, not a pin)
    ref = x[rows].astype(np.float64) @ w.astype(np.float64).T
    rel = np.linalg.norm(y.float().cpu().numpy()[rows] - ref) / np.linalg.norm(ref)
    G.say("  relative error against the unquantised product: %.4f" % rel)
    assert rel < 0.03
