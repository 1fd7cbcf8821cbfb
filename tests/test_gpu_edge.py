"""Degenerate and ragged calls on the GPU against the oracle, through both bf16 kernels
(128-row work items and the 256-row ping-pong kernel): no query rows at all, a reference image
with no tokens, one-token frames, a single query row, reference rows only, head_dim 64 with
ragged frame sizes, and rows whose scores spread so far that the ping-pong kernel's fast pass
hands the work item to its exact pass."""
import numpy as np
import pytest

import fa_workloads as W
import gpu_helpers as G
from frame_aligned_attention_amd import binding as B
from gpu_helpers import random_call

pytestmark = pytest.mark.gpu

BR = pytest.mark.parametrize("br", [128, 256], ids=["bm128", "bm256"])


@BR
def test_no_query_rows(br):
    """Reference rows requested but no reference image: an empty grid, FA_OK, nothing written."""
    G.say("case: reference rows only, no reference tokens, block_rows %d" % br)
    c = G.random_call(31, 16, 2, 2, 128, query_rows=4, block_rows=br)
    assert G.run_call(c) == {}


@BR
def test_zero_token_reference_image(br):
    G.say("case: a reference image of 0 tokens beside one of 9 (t0 1), block_rows %d" % br)
    c = G.random_call(32, 20, 3, 2, 128, ref_tokens=[0, 9], ref_t0=[0, 1], block_rows=br)
    G.compare_all(c, G.run_call(c), "zero-token image")


@BR
def test_one_token_frames(br):
    """T = 1: every source range and frame boundary is one key wide."""
    G.say("case: one-token frames, 37 frames, block_rows %d" % br)
    c = G.random_call(33, 1, 37, 2, 128, ref_tokens=[3], ref_t0=[5], block_rows=br)
    G.compare_all(c, G.run_call(c), "one-token frames")


@BR
def test_single_query_row(br):
    G.say("case: one frame of one token, no reference, block_rows %d" % br)
    c = G.random_call(34, 1, 1, 3, 128, block_rows=br)
    G.compare_all(c, G.run_call(c), "single row")


@BR
def test_reference_rows_only(br):
    G.say("case: reference rows only (two images), block_rows %d" % br)
    c = G.random_call(35, 30, 2, 2, 128, ref_tokens=[40, 217], ref_t0=[0, 1], query_rows=4,
                      block_rows=br)
    G.compare_all(c, G.run_call(c), "reference rows")


@BR
def test_head_dim_64_ragged(br):
    G.say("case: head_dim 64, 333-token frames, block_rows %d" % br)
    c = G.random_call(36, 333, 2, 2, 64, ref_tokens=[45], ref_t0=[1], block_rows=br)
    G.compare_all(c, G.run_call(c), "hd64 ragged")


def _score_spread_call(seed, a, br, key_split):
    """Scores far apart within every row: q = a*u + noise, the first 64 keys of every frame of
    the chunk and the source and of the reference image k = -a*u + noise, all other keys
    k = a*u + noise (u a random sign vector), so each row's first tile scores about -128 a^2
    and later tiles +128 a^2."""
    T, C, H, D = 192, 2, 2, 128
    c = random_call(seed, T, C, H, D, ref_tokens=[128], ref_t0=[0], block_rows=br,
                    key_split=key_split)
    g = np.random.default_rng(seed + 1)
    u = np.where(g.random((H, D)) < 0.5, -1.0, 1.0).astype(np.float32)
    noise = lambda x: W.round_bf16(a * u + 0.5 * x)

    def keys(k, frame_len):
        pos = np.arange(k.shape[0]) % frame_len
        out = noise(k)
        low = pos < 64
        out[low] = W.round_bf16(-a * u + 0.5 * k[low])
        return out

    for kind in c.q:
        c.q[kind] = noise(c.q[kind])
    c.k_hist = keys(c.k_hist, T)
    c.k_src = keys(c.k_src, T)
    c.k_ref = keys(c.k_ref, 128)
    return c


@BR
@pytest.mark.parametrize("a", [2.0, 1.5], ids=["overflow", "sum2e64"])
def test_score_spread_exact_pass(br, a):
    """A row whose first tile scores ~c*256 a^2 (log2 units) below its later tiles: with a = 2
    the ping-pong kernel's fast pass, whose exp offset is the first tile's max, overflows
    (p ~ 2^130) and with a = 1.5 its row sums pass 2^64; either way the workgroup vote reruns the
    item with the row max on every tile.  Compared with the oracle like any call (key split off,
    so every item's first tile is a low one)."""
    G.say("case: score spread a=%g, block_rows %d" % (a, br))
    c = _score_spread_call(41, a, br, B.FA_KEY_SPLIT_OFF)
    res = G.run_call(c)
    ref = G.oracle_all(c)
    for k, (o, lse) in res.items():
        assert np.isfinite(o).all() and np.isfinite(lse).all(), k
        # a handful of keys carry each row's mass (their scores spread over ~10 in log2
        # units), so the LSE bound is the one-key cap (count 1), not the N(0,1) one
        G.tol_check(o, ref[k][0], "bf16", "score spread a=%g %s rows" % (a, G.KIND_NAMES[k]),
                    lse, ref[k][1], counts=np.ones((1, lse.shape[1])))
