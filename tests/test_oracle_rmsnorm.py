"""Pins of the RMSNorm oracle: closed-form rows, numpy fp64 under an error
bound, tails, and row independence."""
import numpy as np
import pytest

import oracle
from tolerance import bits_to_f64, bound_vs_exact, gamma


def rand_bf16(shape, seed, mean=0.0, std=1.0):
    rng = np.random.default_rng(seed)
    f = (rng.standard_normal(shape) * std + mean).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_of(v):
    return np.array([oracle.f32_to_bf16(float(t)) for t in np.ravel(v)], np.uint16).reshape(np.shape(v))


def test_zero_row_gives_zero():
    H = 4096
    x = np.zeros((2, H), np.uint16)
    g = rand_bf16((H,), 1, mean=1.0, std=0.1)
    y, r = oracle.rmsnorm(x, g, 1e-5, return_rinv=True)
    assert np.all(bits_to_f64(y) == 0.0)
    eps = np.float32(1e-5)
    assert r[0] == np.float32(1.0) / np.sqrt(eps)


def test_pm_one_row_closed_form():
    """x = +-1: sum of squares is exactly H, mean exactly 1, so
    r = 1/sqrt(1 + eps) in fp32 and y = bf16((x*r)*g)."""
    H = 4096
    rng = np.random.default_rng(3)
    signs = rng.choice([-1.0, 1.0], size=(1, H)).astype(np.float32)
    x = (signs.view(np.uint32) >> 16).astype(np.uint16)
    g = rand_bf16((H,), 2, mean=1.0, std=0.1)
    y, r = oracle.rmsnorm(x, g, 1e-5, return_rinv=True)
    r32 = np.float32(1.0) / np.sqrt(np.float32(1.0) + np.float32(1e-5))
    assert r[0] == r32
    gf = bits_to_f64(g).astype(np.float32)
    expect = bf16_of((signs[0] * r32) * gf)
    np.testing.assert_array_equal(y[0], expect)


@pytest.mark.parametrize("H", [8, 64, 2048, 4096, 4104, 5000 // 8 * 8, 14336])
def test_within_bound_of_numpy_fp64(H):
    M = 3
    x = rand_bf16((M, H), seed=H)
    g = rand_bf16((H,), seed=H + 1, mean=1.0, std=0.1)
    eps = 1e-5
    xf, gf = bits_to_f64(x), bits_to_f64(g)
    ref = xf / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + eps) * gf
    exact = oracle.rmsnorm_exact(x, g, eps)
    np.testing.assert_allclose(exact, ref, rtol=1e-12, atol=0)
    y = oracle.rmsnorm(x, g, eps)
    # relative error of r: half the sum-tree depth (square root halves it) plus
    # the divide-by-H, +eps, sqrt and reciprocal; then two products.
    depth = 8 * -(-H // 2048) + 6 + 3
    rel = 0.5 * gamma(depth) + gamma(6)
    assert not bound_vs_exact(y, ref, rel * np.abs(ref)).any()


def test_wrong_gain_index_would_fail():
    """Plant a mistake in a reference (gain reversed) and check the bound
    above would see it."""
    H = 256
    x = rand_bf16((1, H), seed=9)
    g = rand_bf16((H,), seed=10, mean=1.0, std=0.1)
    xf, gf = bits_to_f64(x), bits_to_f64(g)
    broken = xf / np.sqrt(np.mean(xf * xf) + 1e-5) * gf[::-1]
    y = oracle.rmsnorm(x, g)
    assert bound_vs_exact(y, broken, 1e-6 * np.abs(broken)).any()


def test_row_independence():
    H = 4096
    x = rand_bf16((64, H), seed=21)
    g = rand_bf16((H,), seed=22, mean=1.0, std=0.1)
    full = oracle.rmsnorm(x, g)
    for M in (1, 3, 8, 31, 64):
        np.testing.assert_array_equal(oracle.rmsnorm(x[:M], g), full[:M])
    np.testing.assert_array_equal(oracle.rmsnorm(x[40:41], g)[0], full[40])
