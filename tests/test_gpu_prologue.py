"""QK prologue (RMSNorm + three-axis RoPE) on the GPU against the oracle, and the prologue fused
with the low-bit quantiser against the unfused kernels (bit-identical) and the oracle.

Tolerance of the bf16 output: |d| <= 2^-8 |ref| + 1e-3 |pair|, with |pair| the magnitude of
the rotated pair (a rotation invariant): the device rounds once to bf16 (2^-9 relative), takes
the angle in fp32 turns (error ~ |turns| * 2^-24, 2e-4 rad at t = 3000) and uses v_sin / v_cos."""
import numpy as np
import pytest
import torch

import gpu_helpers as G
from frame_aligned_attention_amd import binding as B
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def positions(n, seed, t_max=60):
    """(t, y, x) of n tokens laid out frame by frame on a 30 x 52 grid, with a random frame
    offset below t_max."""
    g = np.random.default_rng(seed)
    p = np.arange(n)
    t0 = int(g.integers(0, t_max))
    return np.stack([t0 + p // 1560, (p % 1560) // 52, p % 52], 1).astype(np.int32)


def inputs(seed, n, H, D, b=1):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((b, n, H, D)) * np.exp(g.standard_normal((b, n, H, 1)))).astype(np.float32)
    x = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    gamma = g.uniform(0.5, 1.5, D).astype(np.float32)
    return x, gamma


def check_against_oracle(got, x, gamma, pos, eps, what):
    b = x.shape[0]
    for bi in range(b):
        ref = O.norm_rope(x[bi], gamma, eps, pos).astype(np.float64)
        D = ref.shape[-1]
        P = D // 2
        pair = np.sqrt(ref[..., :P] ** 2 + ref[..., P:] ** 2)
        pair = np.concatenate([pair, pair], -1)
        err = np.abs(got[bi].astype(np.float64) - ref)
        tol = 2.0 ** -8 * np.abs(ref) + 1e-3 * pair
        G.say("  %s batch %d: max|d| %.3g, max|d|/tol %.3f" % (what, bi, err.max(), (err / tol).max()))
        assert np.all(err <= tol), what


CASES = [  # tokens, heads, head_dim, batch, t_max, in place
    (37, 3, 128, 1, 60, False),
    (300, 2, 64, 2, 60, False),
    (4680, 2, 128, 1, 3000, True),
]


@pytest.mark.parametrize("case", CASES, ids=["n%d_h%d_d%d_b%d" % c[:4] for c in CASES])
def test_norm_rope_against_oracle(case):
    n, H, D, b, tmax, inplace = case
    G.say("case: norm + rope %s" % (case,))
    x, gamma = inputs(n + D, n, H, D, b)
    pos = positions(n, n, tmax)
    # batch 2 goes through a strided view: every other token of a twice-longer buffer
    xd = torch.from_numpy(x).to("cuda").to(torch.bfloat16)
    if b > 1:
        big = torch.zeros((b, 2 * n, H, D), dtype=torch.bfloat16, device="cuda")
        big[:, ::2] = xd
        xd = big[:, ::2]
    out = xd if inplace else torch.full_like(xd, float("nan"))
    gd = torch.from_numpy(gamma).cuda()
    pd = torch.from_numpy(pos).cuda()
    B.fa_qk_norm_rope(xd, out, gd, pd, eps=1e-6)
    torch.cuda.synchronize()
    check_against_oracle(out.float().cpu().numpy(), x, gamma, pos, 1e-6, "norm+rope")


@pytest.mark.parametrize("is_key", [False, True], ids=["q", "k"])
def test_fused_quant_equals_unfused(is_key):
    """fa_qk_norm_rope_quant against fa_qk_norm_rope then fa_quantize_lowbit (given mean):
    codes, scales and the query LSE shift bit-identical; codes within one step of the oracle's
    (norm + RoPE in double, rounded to bf16, quantised)."""
    n, H, D = 300, 2, 128
    G.say("case: fused prologue + quantiser, %s, n=%d" % ("keys" if is_key else "queries", n))
    x, gamma = inputs(77 + int(is_key), n, H, D)
    pos = positions(n, 5)
    g = np.random.default_rng(9)
    mean = (0.3 * g.standard_normal((1, H, D))).astype(np.float32)
    xd = torch.from_numpy(x).to("cuda").to(torch.bfloat16)
    gd, pd = torch.from_numpy(gamma).cuda(), torch.from_numpy(pos).cuda()
    md = torch.from_numpy(mean).cuda()
    nb = (n + 127) // 128
    # fused
    codes = torch.zeros((1, n, H, D), dtype=torch.int8, device="cuda")
    scales = torch.zeros((1, H, nb), dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, H, n), dtype=torch.float32, device="cuda") if not is_key else None
    B.fa_qk_norm_rope_quant(xd, codes, scales, gd, pd, is_key, k_mean=md, lse_shift=lse, eps=1e-6)
    # unfused: the bf16 prologue, then the low-bit quantiser of a one-frame call whose target
    # queries (or keys) are that tensor
    y = torch.empty_like(xd)
    B.fa_qk_norm_rope(xd, y, gd, pd, eps=1e-6)
    d = B.make_desc(1, n, H, D, chunk_start=0, query_rows=B.FA_Q_TARGET, dtype=B.FA_LOWBIT)
    L = B.fa_layout_build(d)
    z = torch.zeros_like(xd)
    t = {"q_tgt": z, "k_tgt": z, "v_tgt": z, "k_src": z, "v_src": z}
    t["k_tgt" if is_key else "q_tgt"] = y
    cq = {k: torch.zeros(v.shape, dtype=torch.uint8 if k.startswith("v_") else torch.int8,
                         device="cuda") for k, v in t.items()}
    sq = {k: torch.zeros((1, H, nb), dtype=torch.float32, device="cuda") for k in t}
    lse2 = torch.zeros((1, H, n), dtype=torch.float32, device="cuda")
    kmean = md.clone()
    vmax = torch.zeros((1, H), dtype=torch.float32, device="cuda")
    io_in = B.make_io(t)
    io_out = B.make_io({**cq, "lse_tgt": lse2, "k_mean": kmean, "v_absmax": vmax}, sq)
    B.fa_quantize_lowbit(L, io_in, io_out, B.FA_QUANT_MEAN_GIVEN)
    torch.cuda.synchronize()
    name = "k_tgt" if is_key else "q_tgt"
    assert torch.equal(codes, cq[name]), "codes"
    assert torch.equal(scales, sq[name]), "scales"
    if not is_key:
        assert torch.equal(lse, lse2), "LSE shift"
    # oracle: double prologue, bf16 rounding, then the oracle quantiser
    ref = O.norm_rope(x[0], gamma, 1e-6, pos)
    ref = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    oc, osc = O.quant_int8(ref, mean=mean[0] if is_key else None)
    got = codes.cpu().numpy()[0]
    diff = np.abs(got.astype(np.int32) - oc.astype(np.int32))
    G.say("  codes equal to the oracle's: %.4f, max |d| %d" % ((diff == 0).mean(), diff.max()))
    assert diff.max() <= 1 and (diff == 0).mean() > 0.99
    np.testing.assert_allclose(scales.cpu().numpy()[0], osc, rtol=2.0 ** -7)
