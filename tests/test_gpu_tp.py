"""The local halves of tensor-parallel GEMMs on one GPU.  Row-parallel
(K-sharded): each rank's segment sums, gathered in rank order and folded,
give bi_gemm's bits for 1, 2, 4 and 8 ranks, with even and uneven
(segment-aligned) shards.  Column-parallel (N-sharded): a rank's columns are
bitwise the unsharded columns.  The gather itself is a concatenation here;
across GPUs it is an all-gather of the same bytes."""
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


def sharded(gpu, x, W, seg_counts):
    """Fold of the per-rank segment sums; rank r owns seg_counts[r] segments."""
    parts, k = [], 0
    K = x.shape[1]
    for n in seg_counts:
        k1 = min(K, k + 512 * n)
        parts.append(gpu.gemm_segments(x[:, k:k1].contiguous(), W[k:k1].contiguous()))
        k = k1
    assert k == K
    return gpu.gemm_fold(torch.cat(parts, 0).contiguous())


@pytest.mark.parametrize("M", [1, 16, 40, 200, 1024, 2048])
def test_row_parallel_equals_unsharded(gpu, M):
    x, W = synth.gemm_inputs(M, 4096, 4096, seed=M, w_std=0.02, device=DEV)
    full = gpu.gemm(x, W)
    for ranks in (1, 2, 4, 8):
        y = sharded(gpu, x, W, [8 // ranks] * ranks)
        torch.cuda.synchronize()
        assert same_bits(y, full), f"M={M} ranks={ranks}"


def test_row_parallel_uneven_down_projection(gpu):
    """down 14336 -> 4096: 28 segments over 8 ranks as 4,4,4,4,3,3,3,3, and
    a ragged K whose last segment is short (K = 14336 - 96)."""
    for K, counts in ((14336, [4, 4, 4, 4, 3, 3, 3, 3]), (14336 - 96, [4, 4, 4, 4, 3, 3, 3, 3])):
        x, W = synth.gemm_inputs(16, K, 4096, seed=K, w_std=0.02, device=DEV)
        full = gpu.gemm(x, W)
        y = sharded(gpu, x, W, counts)
        torch.cuda.synchronize()
        assert same_bits(y, full), K


def test_segment_sums_against_oracle_and_fold(gpu):
    """Each segment sum is the oracle's GEMM of that K range within 2 bf16
    ulp once rounded, and the fold of the segments is bi_gemm."""
    x, W = synth.gemm_inputs(8, 1536, 1024, seed=3, w_std=0.02)
    xd, Wd = x.to(DEV), W.to(DEV)
    part = gpu.gemm_segments(xd, Wd)
    torch.cuda.synchronize()
    assert tuple(part.shape) == (3, 8, 1024)
    xb, Wb = synth.to_bits(x), synth.to_bits(W)
    for s in range(3):
        seg = part[s].to(torch.bfloat16)
        want = oracle.gemm(np.ascontiguousarray(xb[:, 512 * s:512 * s + 512]),
                           np.ascontiguousarray(Wb[512 * s:512 * s + 512]))
        check_close_bf16(synth.to_bits(seg), want, what=f"segment {s}")
    assert same_bits(gpu.gemm_fold(part), gpu.gemm(xd, Wd))


@pytest.mark.parametrize("M", [1, 300])
def test_column_parallel_equals_unsharded(gpu, M):
    """gate_up 4096 -> 28672 split over 8 ranks by columns (3584 each)."""
    x, W = synth.gemm_inputs(M, 4096, 28672, seed=10 + M, w_std=0.02, device=DEV)
    full = gpu.gemm(x, W)
    for r in range(8):
        y = gpu.gemm(x, W[:, 3584 * r:3584 * (r + 1)].contiguous())
        torch.cuda.synchronize()
        assert same_bits(y, full[:, 3584 * r:3584 * (r + 1)].contiguous()), f"M={M} rank {r}"
