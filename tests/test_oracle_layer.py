"""Pins for the oracle's element-wise decoder-layer steps (RoPE table and
rotation, SiLU-gated product, residual add): closed forms, identities and
planted tables that a sign, index or half-swap mistake would fail."""
import math

import numpy as np
import pytest

import oracle

D = 128
HALF = D // 2


def bf16_bits(values) -> np.ndarray:
    """Exact bf16 values (the low 16 fp32 bits must be zero) as bits."""
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF)
    return (u >> 16).astype(np.uint16)


def bits_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def rand_bf16(shape, seed, scale=1.0):
    f = (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)
    u = f.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_rope_table_closed_forms():
    c, s = oracle.rope_table(5e5, D, 4)
    assert np.all(c[0] == 1.0) and np.all(s[0] == 0.0)          # angle 0
    # column 0 has inverse frequency theta^0 = 1, so the angle is the position
    assert c[1, 0] == np.float32(0.5403023058681398)              # cos 1
    assert s[1, 0] == np.float32(0.8414709848078965)              # sin 1
    assert c[3, 0] == np.float32(-0.9899924966004454)             # cos 3
    assert s[3, 0] == np.float32(0.1411200080598672)              # sin 3


def test_rope_table_identities():
    c, s = oracle.rope_table(5e5, D, 2048)
    c64, s64 = c.astype(np.float64), s.astype(np.float64)
    # cos^2 + sin^2 = 1 up to the two fp32 roundings
    assert np.max(np.abs(c64 ** 2 + s64 ** 2 - 1.0)) < 4 * 2.0 ** -24
    # angle addition: entries for a + b from the entries for a and b
    for a, b in ((1, 1), (7, 30), (500, 1000), (1023, 1024)):
        ca = c64[a] * c64[b] - s64[a] * s64[b]
        sa = s64[a] * c64[b] + c64[a] * s64[b]
        assert np.max(np.abs(ca - c64[a + b])) < 1e-6, (a, b)
        assert np.max(np.abs(sa - s64[a + b])) < 1e-6, (a, b)
    # frequencies fall with the column index: the angle of column i at
    # position p is p * theta^(-2i/D), so the last column turns slowest
    i = HALF - 1
    ang = math.atan2(s64[1000, i], c64[1000, i])
    assert abs(ang - 1000 * 5e5 ** (-2 * i / D)) < 1e-6


def test_rope_position_zero_is_identity():
    c, s = oracle.rope_table(5e5, D, 8)
    x = rand_bf16((5, 4 * D), seed=1)
    y = oracle.rope(x, np.zeros(5, np.int32), 4, D, c, s)
    np.testing.assert_array_equal(y.reshape(5, -1), x)


def test_rope_quarter_turn_table_swaps_halves():
    """With cos = 0 and sin = 1 every pair (a, b) goes to (-b, a) exactly; a
    swapped sign or a wrong partner index fails this."""
    c = np.zeros((2, HALF), np.float32)
    s = np.ones((2, HALF), np.float32)
    x = rand_bf16((3, 2 * D), seed=2)
    y = oracle.rope(x, np.ones(3, np.int32), 2, D, c, s)
    xf = bits_f32(x).reshape(3, 2, D)
    yf = bits_f32(y)
    np.testing.assert_array_equal(yf[..., :HALF], -xf[..., HALF:])
    np.testing.assert_array_equal(yf[..., HALF:], xf[..., :HALF])


def test_rope_preserves_pair_norms_and_reads_strided_rows():
    c, s = oracle.rope_table(5e5, D, 4096)
    M = 6
    pos = np.array([0, 1, 17, 255, 2048, 4095], np.int32)
    row = rand_bf16((M, 3 * D + 64), seed=3)       # 3 heads, then unrelated values
    y = oracle.rope(row, pos, 3, D, c, s)
    x = bits_f32(row)[:, :3 * D].reshape(M, 3, D).astype(np.float64)
    yf = bits_f32(y).astype(np.float64)
    n_in = x[..., :HALF] ** 2 + x[..., HALF:] ** 2
    n_out = yf[..., :HALF] ** 2 + yf[..., HALF:] ** 2
    # two bf16 roundings per output: relative error of a norm < 2 * 2^-8
    assert np.all(np.abs(n_out - n_in) <= 2 * 2.0 ** -7 * n_in + 1e-30)
    # exact per-element form in fp32 (products, then the sum), one bf16 rounding
    cp, sp = c[pos][:, None, :], s[pos][:, None, :]
    xa, xb = x[..., :HALF].astype(np.float32), x[..., HALF:].astype(np.float32)
    lo = (xa * cp - xb * sp).astype(np.float32)
    hi = (xb * cp + xa * sp).astype(np.float32)
    want = np.concatenate([lo, hi], axis=-1)
    u = want.view(np.uint32)
    want_bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(y, want_bits)


def test_silu_mul_special_values():
    F = 4
    gate = [0.0, 100.0, -100.0, 2.0]
    up = [5.0, 3.0, 3.0, 0.0]
    y = bits_f32(oracle.silu_mul(bf16_bits([gate + up]))[0])
    assert y[0] == 0.0                      # silu(0) = 0
    assert y[1] == 300.0                    # silu(100) = 100 in fp32
    assert y[2] == 0.0 or abs(y[2]) < 1e-38  # silu(-100) ~ -3.7e-42
    assert y[3] == 0.0                      # up = 0
    # the gate is the first half: swapping the halves changes the value
    a = bits_f32(oracle.silu_mul(bf16_bits([[2.0, 3.0]]))[0])[0]
    b = bits_f32(oracle.silu_mul(bf16_bits([[3.0, 2.0]]))[0])[0]
    assert a != b
    assert abs(a - 3.0 * 2.0 / (1.0 + math.exp(-2.0))) < 2.0 ** -7 * 6


def test_silu_mul_matches_fp64_definition():
    gu = rand_bf16((32, 2 * 256), seed=4, scale=3.0)
    y = bits_f32(oracle.silu_mul(gu)).astype(np.float64)
    g = bits_f32(gu[:, :256]).astype(np.float64)
    u = bits_f32(gu[:, 256:]).astype(np.float64)
    exact = g / (1.0 + np.exp(-g)) * u
    # four fp32 roundings and one bf16 rounding
    tol = 2.0 ** -8 * np.abs(exact) + 8 * 2.0 ** -24 * np.abs(exact) + 1e-38
    assert np.all(np.abs(y - exact) <= tol)


def test_add_is_one_rounding_of_the_exact_sum():
    a = bf16_bits([1.0, 1.0, -2.0, 0.5, 3.0])
    b = bf16_bits([2.0 ** -8, 3 * 2.0 ** -8, 2.0, 0.25, -1.0])
    y = bits_f32(oracle.add(a, b))
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even wins; 1 + 3*2^-8 rounds up
    np.testing.assert_array_equal(y, np.array([1.0, 1.0 + 2.0 ** -6, 0.0, 0.75, 2.0], np.float32))
    x1, x2 = rand_bf16((1000,), 5), rand_bf16((1000,), 6)
    s = (bits_f32(x1).astype(np.float64) + bits_f32(x2).astype(np.float64)).astype(np.float32)
    u = s.view(np.uint32)
    np.testing.assert_array_equal(oracle.add(x1, x2), ((u + 0x7FFF + ((u >> 16) & 1)) >> 16)
                                  .astype(np.uint16))
