"""bi_rmsnorm on the GPU: bit-exact with the oracle (every step is an IEEE
basic operation in the same order), bitwise across M, and the fast twin."""
import numpy as np
import pytest
import torch

import oracle
from invariant_bi_gemm_02_amd import synth
from tolerance import check_close_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_config2_bitwise_across_m_and_exact_vs_oracle(gpu):
    H = 4096
    x, g = synth.rmsnorm_inputs(512, H, seed=1, device=DEV)
    full = gpu.rmsnorm(x, g, 1e-5)
    for M in synth.RMSNORM_M:
        y = gpu.rmsnorm(x[:M].contiguous(), g, 1e-5)
        assert same_bits(y, full[:M]), f"M={M}"
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(synth.to_bits(x), synth.to_bits(g), 1e-5)
    np.testing.assert_array_equal(synth.to_bits(full), ref)


@pytest.mark.parametrize("M,H", [(1, 8), (3, 64), (5, 2048), (2, 4104), (4, 14336), (9, 5000 // 8 * 8)])
def test_other_widths_exact(gpu, M, H):
    x, g = synth.rmsnorm_inputs(M, H, seed=H, device=DEV)
    y = gpu.rmsnorm(x, g, 1e-6)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(synth.to_bits(y),
                                  oracle.rmsnorm(synth.to_bits(x), synth.to_bits(g), 1e-6))


def test_zero_row(gpu):
    x = torch.zeros((2, 4096), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(4096, dtype=torch.bfloat16, device=DEV)
    y = gpu.rmsnorm(x, g)
    torch.cuda.synchronize()
    assert torch.all(y.float() == 0)


@pytest.mark.parametrize("M", [1, 512, 2048])
def test_fast_twin(gpu, M):
    x, g = synth.rmsnorm_inputs(M, 4096, seed=7, device=DEV)
    y = gpu.rmsnorm_fast(x, g)
    torch.cuda.synchronize()
    rows = sorted(set([0, M // 2, M - 1]))
    ref = oracle.rmsnorm(synth.to_bits(x[rows]), synth.to_bits(g))
    check_close_bf16(synth.to_bits(y[rows]), ref, what=f"rmsnorm fast M={M}")
