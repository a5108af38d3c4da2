"""The measurement helpers on the GPU: the streaming read touches every word
of its buffer exactly once (the XOR of its per-wave words equals the XOR of
the buffer's words), and the matrix-core loop is finite and repeatable."""
import numpy as np
import pytest
import torch

import invariant_bi_gemm_02_amd as bi

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [16, 1040, (1 << 20) + 48, 64 << 20])
def test_ceiling_read_reads_every_word_once(gpu, nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to(DEV)
    out = torch.zeros(bi.CEILING_READ_OUT_WORDS, dtype=torch.int32, device=DEV)
    bi.ceiling_read(buf, out=out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want


def test_ceiling_mfma_is_finite_and_repeatable(gpu):
    a, flops = bi.ceiling_mfma(100, 64)
    b, _ = bi.ceiling_mfma(100, 64)
    torch.cuda.synchronize()
    assert flops == 64 * 4 * 100 * 8 * 16384
    assert torch.isfinite(a).all()
    assert torch.equal(a, b)
