"""Pins of the GEMM oracle against things other than itself.

* the fp32 associativity example the Determinism article prints (section 2.1);
* bf16-exact operands that make every ordering choice of the schedule visible
  (block order, segment start from +0, segment fold order);
* exact-arithmetic inputs (a permutation matrix, small integers);
* numpy's fp64 matmul (a library routine) under the fp32 error bound;
* row independence (the oracle's own M-invariance).
"""
import json
import os

import numpy as np
import pytest

import oracle
from tolerance import bits_to_f64, bound_vs_exact, gamma, gemm_depth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16_bits(values) -> np.ndarray:
    """bf16 bits of values that are exactly representable in bf16."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value not exactly representable in bf16")
    return (u >> 16).astype(np.uint16)


def rand_bf16(shape, seed, std=1.0):
    rng = np.random.default_rng(seed)
    f = (rng.standard_normal(shape) * std).astype(np.float32)
    # truncate to bf16 (any rounding is fine for inputs: both sides get the same bits)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_fold_matches_page_example():
    with open(os.path.join(GOLDEN, "fp32_assoc_example.json")) as fh:
        g = json.load(fh)
    a, b, c = (np.float32(g["operands"][k]) for k in ("a", "b", "c"))
    assert oracle.fold_f32([a, b, c]) == g["left_grouping"]["printed"]
    assert oracle.fold_f32([a, oracle.fold_f32([b, c])]) == g["right_grouping"]["printed"]


# Products 2^26, -2^26 and 1: the left fold gives exactly 1 (2^26 - 2^26 = 0
# exactly, then 0 + 1), any grouping that adds 1 to 2^26 first gives 0
# (fp32 spacing at 2^26 is 8, so 2^26 + 1 rounds back to 2^26).
BIG = 2.0 ** 13


def one_column_case(K, placements):
    """x[1,K], W[K,2]: column 0 carries the products at the given k positions,
    column 1 is all zero."""
    x = np.zeros((1, K), np.float32)
    w = np.zeros((K, 2), np.float32)
    for k, (xv, wv) in placements.items():
        x[0, k] = xv
        w[k, 0] = wv
    return bf16_bits(x), bf16_bits(w)


@pytest.mark.parametrize("ks,expect", [
    ((0, 512, 1024), 1.0),   # three segments, folded 0,1,2
    ((1024, 512, 0), 0.0),   # the same products, 1 now in the first segment
    ((0, 32, 64), 1.0),      # three K-blocks of one segment, in block order
    ((64, 32, 0), 0.0),
])
def test_gemm_order_across_blocks_and_segments(ks, expect):
    K = 1536
    vals = [(BIG, BIG), (-BIG, BIG), (1.0, 1.0)]
    x, w = one_column_case(K, dict(zip(ks, vals)))
    y, y32 = oracle.gemm(x, w, return_f32=True)
    assert y32[0, 0] == expect
    assert y32[0, 1] == 0.0
    assert bits_to_f64(y)[0, 0] == expect


def test_gemm_segment_starts_from_zero():
    """Segment 1 holds -2^26 then +1 in two of its blocks.  Accumulated from +0
    it is -(2^26 - 1), which rounds to -2^26, so the fold gives 0.  A schedule
    that carried the running sum into segment 1 would give 1."""
    K = 1024
    x, w = one_column_case(K, {0: (BIG, BIG), 512: (-BIG, BIG), 544: (1.0, 1.0)})
    _, y32 = oracle.gemm(x, w, return_f32=True)
    assert y32[0, 0] == 0.0


def test_gemm_inblock_model_is_left_to_right():
    """Inside one K-block the oracle models the 32 products as a left-to-right
    sum: (1 + 2^26) - 2^26 = 0.  This is a model of the matrix core, not a
    pinned fact about it."""
    K = 32
    x, w = one_column_case(K, {0: (1.0, 1.0), 1: (BIG, BIG), 2: (-BIG, BIG)})
    _, y32 = oracle.gemm(x, w, return_f32=True)
    assert y32[0, 0] == 0.0


@pytest.mark.parametrize("K", [32, 96, 544, 1024])
def test_gemm_permutation_is_exact(K):
    rng = np.random.default_rng(K)
    N = K
    perm = rng.permutation(K)
    w = np.zeros((K, N), np.float32)
    w[perm, np.arange(N)] = 1.0
    x = rand_bf16((3, K), seed=K)
    y = oracle.gemm(x, bf16_bits(w))
    np.testing.assert_array_equal(y, x[:, perm])


@pytest.mark.parametrize("K", [64, 1024, 1536])
def test_gemm_small_integers_are_exact(K):
    rng = np.random.default_rng(7 + K)
    x = rng.integers(-3, 4, size=(4, K)).astype(np.float32)
    w = rng.integers(-3, 4, size=(K, 48)).astype(np.float32)
    ref = x.astype(np.float64) @ w.astype(np.float64)
    y, y32 = oracle.gemm(bf16_bits(x), bf16_bits(w), return_f32=True)
    np.testing.assert_array_equal(y32.astype(np.float64), ref)
    ref_bits = np.array([oracle.f32_to_bf16(float(v)) for v in ref.ravel()],
                        np.uint16).reshape(ref.shape)
    np.testing.assert_array_equal(y, ref_bits)


@pytest.mark.parametrize("M,N,K", [(1, 16, 32), (2, 64, 96), (4, 40, 512), (3, 64, 544),
                                   (4, 33, 1024), (2, 17, 1536)])
def test_gemm_within_fp32_bound_of_numpy_fp64(M, N, K):
    x = rand_bf16((M, K), seed=M * 1000 + K)
    w = rand_bf16((K, N), seed=N * 7 + K)
    ref = bits_to_f64(x) @ bits_to_f64(w)          # library fp64 matmul
    exact = oracle.gemm_exact(x, w)
    np.testing.assert_allclose(exact, ref, rtol=0, atol=1e-9)
    A = np.abs(bits_to_f64(x)) @ np.abs(bits_to_f64(w))
    np.testing.assert_allclose(oracle.gemm_absdot(x, w), A, rtol=1e-12)
    err = gamma(gemm_depth(K)) * A
    y, y32 = oracle.gemm(x, w, return_f32=True)
    assert np.all(np.abs(y32.astype(np.float64) - ref) <= err)
    assert not bound_vs_exact(y, ref, err).any()


def test_gemm_dropped_term_would_fail_the_bound():
    """Plant a mistake on the CPU side: drop one product from the reference
    and check the bound used above notices it."""
    M, N, K = 2, 32, 544
    x = rand_bf16((M, K), seed=11)
    w = rand_bf16((K, N), seed=12)
    xf, wf = bits_to_f64(x), bits_to_f64(w)
    ref = xf @ wf
    broken = ref - xf[:, 100:101] * wf[100:101, :]
    A = np.abs(xf) @ np.abs(wf)
    y = oracle.gemm(x, w)
    assert bound_vs_exact(y, broken, gamma(gemm_depth(K)) * A).any()


def test_gemm_row_independence():
    K, N = 1088, 48
    x = rand_bf16((33, K), seed=5)
    w = rand_bf16((K, N), seed=6, std=0.02)
    full = oracle.gemm(x, w)
    for M in (1, 2, 7, 16, 33):
        part = oracle.gemm(x[:M], w)
        np.testing.assert_array_equal(part, full[:M])
    for i in (0, 5, 32):
        np.testing.assert_array_equal(oracle.gemm(x[i:i + 1], w)[0], full[i])


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    assert oracle.f32_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> up
    assert oracle.f32_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.f32_to_bf16(-2.5) == 0xC020
    nan = oracle.f32_to_bf16(float("nan"))
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0
