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
