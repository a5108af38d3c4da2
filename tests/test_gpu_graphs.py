"""HIP graph capture of library calls: replays give the eager bits, also after
the binding's scratch buffers would have been replaced.

torch captures every graph on one shared capture stream and empties its
memory cache before each capture.  The binding's per-stream scratch buffer
therefore used to outlive the graph it was allocated in: a later capture
could start on it and, growing it for a larger call, free it while its own
earlier captured kernels still held its address; the next capture's cache
flush then released that memory and the replays wrote to unmapped memory.
Calls under capture now take a scratch buffer of the graph's own pool, which
lives as long as the graph."""
import pytest
import torch

from invariant_bi_gemm_02_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    return g, out


def test_replays_after_scratch_growth_and_later_capture(gpu):
    x1, w1 = synth.gemm_inputs(1, 4096, 4096, seed=60, device=DEV)      # 8 segments, 128 KB
    x2, w2 = synth.gemm_inputs(16, 4096, 28672, seed=61, device=DEV)    # 8 segments, 14.7 MB
    ref1, ref2 = gpu.gemm(x1, w1), gpu.gemm(x2, w2)
    torch.cuda.synchronize()

    g1, _ = capture(lambda: gpu.gemm(x1, w1))      # scratch first taken under capture
    del g1
    # the small call first, then one that needs more scratch than any before
    g2, (y1, y2) = capture(lambda: (gpu.gemm(x1, w1), gpu.gemm(x2, w2)))
    g3, y3 = capture(lambda: gpu.gemm(x1, w1))     # torch empties its cache first
    for _ in range(3):
        g2.replay()
        torch.cuda.synchronize()
        assert same_bits(y1, ref1) and same_bits(y2, ref2)
        y1.zero_()
        y2.zero_()
        assert same_bits(gpu.gemm(x2, w2), ref2)   # eager work between the replays
        torch.cuda.synchronize()
    g3.replay()
    torch.cuda.synchronize()
    assert same_bits(y3, ref1)


def test_tiny_decoder_graph_replays(gpu):
    """The whole forward and the sampler, captured twice in a row: a decode
    step (one row per request, per-row attention) and a grouped window
    (multi-query attention with split chunks) followed by sampling.  Every
    replay, with eager work and synchronizations between the replays, gives
    the eager logits and tokens bit for bit."""
    import numpy as np
    from invariant_bi_gemm_02_amd.decoder import Decoder

    cfg = synth.TINY
    w = synth.decoder_weights(cfg, seed=62, device=DEV)
    req = synth.Requests([40, 17, 29], max_len=96, vocab=cfg.vocab, page_size=16, seed=63)
    dec = Decoder(cfg, w, req.num_pages, 128, DEV)
    segs = [(r, np.arange(n), req.prompts[r]) for r, n in enumerate(req.prompt_lens)]
    dec.run(dec.prepare(*synth.grouped_rows(req, segs)))       # prompts into the KV cache
    rid = np.arange(3)
    pos = np.array(req.prompt_lens, np.int32)
    tok = np.array([5, 77, 901], np.int32)
    step_rows = dec.prepare(*req.rows(rid, pos, tok))
    win = [(r, np.arange(pos[r], pos[r] + n), (np.arange(n) * 31 + r) % cfg.vocab)
           for r, n in enumerate((6, 2, 9))]
    win_rows = dec.prepare(*synth.grouped_rows(req, win))
    M = 17
    seeds = torch.from_numpy(np.arange(1000, 1000 + M, dtype=np.uint64)).to(DEV)
    steps = torch.from_numpy(np.full(M, 3, dtype=np.uint64)).to(DEV)
    temps = torch.full((M,), 0.8, dtype=torch.float32, device=DEV)

    def window():
        logits = dec.run(win_rows)
        return logits, gpu.sample(logits, seeds, steps, temps)

    ref_step = dec.run(step_rows)
    ref_win, ref_tok = window()
    torch.cuda.synchronize()
    g_step, out_step = capture(lambda: dec.run(step_rows))
    g_win, (out_win, out_tok) = capture(window)
    for _ in range(3):
        g_step.replay()
        g_win.replay()
        torch.cuda.synchronize()
        assert same_bits(out_step, ref_step) and same_bits(out_win, ref_win)
        assert torch.equal(out_tok, ref_tok)
        out_step.zero_()
        out_win.zero_()
        out_tok.zero_()
        assert same_bits(dec.run(win_rows), ref_win)      # eager work between the replays
        torch.cuda.synchronize()
