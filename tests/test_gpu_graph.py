"""The per-chunk sequence of a stream captured into HIP graphs (quantise -> attention -> ring
append), replayed against eager execution of the same chunks: bit-identical outputs and ring.

A ring of 12 frames and 3-frame chunks repeat their slot pattern every 4 chunks, and once the
ring is full every steady chunk has the same block map; so one graph per phase (captured at
chunks 4..7) replays chunks 4..13.  Between replays the test does its own eager work (copying the
next chunk's inputs into the static buffers) and synchronises, and checks every replay.  At two
heads the bf16 chunk's 38 work items of 256 rows fit one round, so they are split into key parts
and each bf16 graph also holds the merge kernel."""
import pytest
import torch

import fa_workloads as W
import gpu_helpers as G
from frame_aligned_attention_amd import binding as B

pytestmark = pytest.mark.gpu

CHUNKS = 14
FIRST_GRAPH = 4  # chunk_start 12: the ring is full from here on


def nblk(n):
    return (n + 127) // 128


class ChunkSeq:
    """Static buffers of one stream (inputs, outputs, ring, low-bit codes) and the per-chunk
    sequence over them."""

    def __init__(self, H, lowbit):
        self.w = w = W.WORKLOADS[4 if lowbit else 2]
        self.H, self.lowbit = H, lowbit
        T, C, D = w.T, w.C, w.D
        bf = dict(dtype=torch.bfloat16, device="cuda")
        self.inp = {n: torch.zeros((1, C * T, H, D), **bf)
                    for n in ("q_tgt", "k_tgt", "v_tgt", "k_src", "v_src")}
        r = W.ref_tensors(w, H=H)
        self.inp["k_ref"], self.inp["v_ref"] = G.dev(r["k_ref"]), G.dev(r["v_ref"])
        self.inp["k_ring"] = torch.zeros((1, w.cache_frames * T, H, D), **bf)
        self.inp["v_ring"] = torch.zeros((1, w.cache_frames * T, H, D), **bf)
        self.out = {"o_tgt": torch.zeros((1, C * T, H, D), **bf),
                    "lse_tgt": torch.zeros((1, H, C * T), dtype=torch.float32, device="cuda")}
        if lowbit:
            self.codes, self.scales = {}, {}
            for n, x in self.inp.items():
                if n == "q_tgt" or n.startswith(("k_", "v_")):
                    dt = torch.uint8 if n.startswith("v_") else torch.int8
                    self.codes[n] = torch.zeros(x.shape, dtype=dt, device="cuda")
                    self.scales[n] = torch.zeros((1, H, nblk(x.shape[1])), dtype=torch.float32,
                                                 device="cuda")
            self.k_mean = torch.zeros((1, H, D), dtype=torch.float32, device="cuda")
            self.v_absmax = torch.zeros((1, H), dtype=torch.float32, device="cuda")
        self.layouts = {}

    def desc(self, cs):
        w = self.w
        return B.make_desc(w.C, w.T, self.H, w.D, ref_tokens=w.ref_tokens, ref_t0=w.ref_t0,
                           chunk_start=cs, window=w.window, cache_frames=w.cache_frames,
                           query_rows=B.FA_Q_TARGET,
                           dtype=B.FA_LOWBIT if self.lowbit else B.FA_BF16)

    def layout(self, cs):
        if cs not in self.layouts:
            L = B.fa_layout_build(self.desc(cs), max(0, cs - self.w.cache_frames))
            B.fa_layout_prepare(L)
            self.layouts[cs] = L
        return self.layouts[cs]

    def load(self, ch):
        x = W.chunk_tensors(self.w, ch, H=self.H)
        for n in ("q_tgt", "k_tgt", "v_tgt", "k_src", "v_src"):
            self.inp[n].copy_(torch.from_numpy(x[n]).unsqueeze(0).to(torch.bfloat16))

    def run(self, cs, stream=None):
        """The chunk's sequence, launched on `stream` (None: torch's current stream)."""
        L = self.layout(cs)
        if self.lowbit:
            io_in = B.make_io(self.inp)
            io_q = B.make_io({**self.codes, "lse_tgt": self.out["lse_tgt"], "k_mean": self.k_mean,
                              "v_absmax": self.v_absmax}, self.scales)
            B.fa_quantize_lowbit(L, io_in, io_q, 0, stream)
            io = B.make_io({**self.codes, **self.out, "v_absmax": self.v_absmax}, self.scales)
        else:
            io = B.make_io({**self.inp, **self.out})
        B.fa_attn_fwd(L, io, stream)
        B.fa_ring_append(self.desc(cs), self.inp["k_ring"], self.inp["v_ring"], self.inp["k_tgt"],
                         self.inp["v_tgt"], cs, self.w.C, stream)


def block_map(L):
    n, _, _ = B.fa_layout_tiles(L)
    return [B.fa_layout_tile(L, i) for i in range(n)]


@pytest.mark.parametrize("lowbit", [False, True], ids=["bf16", "lowbit"])
def test_graph_replay_matches_eager(lowbit):
    G.say("case: %s stream, 14 chunks, graphs per ring phase from chunk 4" %
          ("low-bit" if lowbit else "bf16"))
    H = 2
    eager, graph = ChunkSeq(H, lowbit), ChunkSeq(H, lowbit)
    C = eager.w.C
    want = {}
    for ch in range(CHUNKS):
        eager.load(ch)
        eager.run(ch * C)
        torch.cuda.synchronize()
        want[ch] = (eager.out["o_tgt"].clone(), eager.out["lse_tgt"].clone())
    graphs = {}
    captured_map = None
    for ch in range(CHUNKS):
        cs = ch * C
        graph.load(ch)
        torch.cuda.synchronize()
        if ch < FIRST_GRAPH:
            graph.run(cs)
        else:
            L = graph.layout(cs)
            if captured_map is None:
                captured_map = block_map(L)
                assert (B.fa_layout_splits(L)[0] == 0) == lowbit, "bf16 items split into parts"
            assert block_map(L) == captured_map, "steady chunks share one block map"
            phase = ch % 4
            if phase not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    graph.run(cs)
                graphs[phase] = g
            graphs[phase].replay()
        torch.cuda.synchronize()
        assert torch.equal(graph.out["o_tgt"], want[ch][0]), "O of chunk %d" % ch
        assert torch.equal(graph.out["lse_tgt"], want[ch][1]), "LSE of chunk %d" % ch
    assert torch.equal(graph.inp["k_ring"], eager.inp["k_ring"])
    assert torch.equal(graph.inp["v_ring"], eager.inp["v_ring"])
    G.say("  %d graphs, chunks %d..%d replayed, bit-identical" % (len(graphs), FIRST_GRAPH,
                                                                   CHUNKS - 1))


def test_capture_without_prepare_is_rejected():
    G.say("case: fa_attn_fwd under capture with a block map not on the device")
    seq = ChunkSeq(1, False)
    L = B.fa_layout_build(seq.desc(0), 0)  # not prepared
    io = B.make_io({**seq.inp, **seq.out})
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g):
        seq.out["lse_tgt"].add_(1.0)  # keep the captured graph non-empty
        try:
            B.fa_attn_fwd(L, io)
        except B.FaError as e:
            err = e
    assert err is not None and "fa_layout_prepare" in str(err)
    g.replay()
    torch.cuda.synchronize()
    assert float(seq.out["lse_tgt"].max()) == 1.0
