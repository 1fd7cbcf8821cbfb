"""Degenerate and ragged calls on the GPU against the oracle, through both bf16 kernels
(128-row work items and the 256-row ping-pong kernel): no query rows at all, a reference image
with no tokens, one-token frames, a single query row, reference rows only, head_dim 64 with
ragged frame sizes."""
import pytest

import gpu_helpers as G

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
