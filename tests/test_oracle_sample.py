"""Pins for the oracle's sampler and commit-or-rollback bookkeeping.
Philox4x64-10 against numpy's Philox bit generator; greedy decoding against
numpy's argmax; the uniforms' range, grid and moments; Gumbel-max token
frequencies against the softmax they must follow; the temperature limits;
worked cases of the commit-or-rollback rule (LLM-42 digest, method)."""
import numpy as np
import pytest

import oracle


def bits_of(f32):
    return (np.asarray(f32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("key", [(0, 0), (123, 456), (2**64 - 1, 7)])
def test_philox_matches_numpy(key):
    rng = np.random.default_rng(sum(key) % 1000)
    for _ in range(5):
        ctr = [int(v) for v in rng.integers(1, 2**63, 4, dtype=np.uint64)]
        # numpy's generator steps its counter before each block
        bg = np.random.Philox(counter=[ctr[0] - 1, ctr[1], ctr[2], ctr[3]],
                              key=np.array(key, np.uint64))
        np.testing.assert_array_equal(oracle.philox4x64(ctr, key), bg.random_raw(4))


def test_uniforms_lie_on_the_half_grid():
    u = np.array([oracle.sample_uniform(99, 3, v) for v in range(40000)], np.float64)
    assert u.min() > 0 and u.max() < 1
    k = u * 2**23 - 0.5
    np.testing.assert_array_equal(k, np.round(k))
    assert abs(u.mean() - 0.5) < 0.01 and abs(u.var() - 1 / 12) < 0.005
    # different steps and seeds give different streams
    assert oracle.sample_uniform(99, 4, 0) != oracle.sample_uniform(99, 3, 0)
    assert oracle.sample_uniform(98, 3, 0) != oracle.sample_uniform(99, 3, 0)


def test_greedy_is_first_argmax():
    rng = np.random.default_rng(1)
    l = rng.standard_normal((6, 300)).astype(np.float32)
    l[1, [7, 50]] = 9.0                      # a tie: the first index wins
    l[2, :] = -np.inf
    l[3, 5] = np.nan                         # NaN never wins
    l[3, 6] = 20.0
    lb = bits_of(l)
    got = oracle.sample(lb, np.arange(6), np.zeros(6), np.zeros(6))
    f = (lb.astype(np.uint32) << 16).view(np.float32)
    want = np.argmax(np.where(np.isnan(f), -np.inf, f), axis=1)
    np.testing.assert_array_equal(got, want)
    assert got[1] == 7 and got[2] == 0 and got[3] == 6


@pytest.mark.parametrize("T", [1.0, 0.5])
def test_gumbel_max_follows_the_softmax(T):
    """Token frequencies over 20000 (seed, step) draws against softmax(l/T):
    chi-square with 4 degrees of freedom far below its 1e-4 quantile (23.5)."""
    l = np.array([1.0, 0.5, 0.0, -1.0, 2.0], np.float32)
    n = 20000
    lb = np.tile(bits_of(l), (n, 1))
    tok = oracle.sample(lb, np.arange(n) * 7919 + 1, np.arange(n) % 13, np.full(n, T))
    freq = np.bincount(tok, minlength=5)
    p = np.exp(l.astype(np.float64) / T)
    p /= p.sum()
    chi2 = float(((freq - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 23.5, (freq, n * p, chi2)


def test_temperature_limits():
    n = 4000
    l = np.array([3.0, 0.0, -2.0, 1.0], np.float32)
    lb = np.tile(bits_of(l), (n, 1))
    # a tiny temperature is greedy for well-separated logits
    tok = oracle.sample(lb, np.arange(n), np.ones(n), np.full(n, 1e-4))
    assert (tok == 0).all()
    # a huge temperature is close to uniform
    tok = oracle.sample(lb, np.arange(n), np.ones(n), np.full(n, 1e4))
    freq = np.bincount(tok, minlength=4) / n
    assert np.abs(freq - 0.25).max() < 0.04


def test_verify_commit_worked_cases():
    # request 0: all 3 candidates match; 1: mismatch at the first; 2: at the
    # third of four; 3: a one-token window that matches; 4: empty window
    cand = np.array([5, 6, 7, 1, 2, 8, 8, 3, 9, 4], np.int32)
    ver = np.array([5, 6, 7, 9, 2, 8, 8, 0, 9, 4], np.int32)
    rs = np.array([0, 3, 5, 9, 10, 10], np.int32)
    L = np.array([10, 20, 30, 40, 50], np.int32)
    acc, new_len, fix = oracle.verify_commit(cand, ver, rs, L)
    # request 2 (rows 5..8): cand 8 8 3 9, ver 8 8 0 9 -> two match, fix 0
    np.testing.assert_array_equal(acc, [3, 0, 2, 1, 0])
    np.testing.assert_array_equal(new_len, [13, 21, 33, 41, 50])
    np.testing.assert_array_equal(fix, [-1, 9, 0, -1, -1])
