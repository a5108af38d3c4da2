"""Pins of the paged decode-attention oracle: one token, constant V, q = 0,
numpy fp64 softmax through an independent gather, chunk-edge lengths, page
layout, batch composition and GQA grouping."""
import numpy as np
import pytest

import oracle
from invariant_bi_gemm_02_amd import synth
from tolerance import bits_to_f64, check_close_bf16

HQ, HKV, D, PS = 8, 2, 128, 16   # small head counts keep the CPU cases quick


def make(ctx, seed, shuffle=True, extra=0, hq=HQ, hkv=HKV):
    q, kv, bt, cl = synth.attn_inputs(ctx, seed, shuffle=shuffle, extra_pages=extra, Hq=hq,
                                      Hkv=hkv)
    return synth.to_bits(q), synth.to_bits(kv), bt, cl


def numpy_reference(q, kv, bt, cl, hkv=HKV):
    """fp64 softmax attention with the gather written by numpy indexing."""
    qf, kvf = bits_to_f64(q), bits_to_f64(kv)
    B, Hq, Dd = qf.shape
    G = Hq // hkv
    out = np.zeros((B, Hq, Dd))
    for b in range(B):
        L = int(cl[b])
        if L <= 0:
            continue
        t = np.arange(L)
        pages = bt[b, t // PS]
        slots = t % PS
        for h in range(Hq):
            K = kvf[pages, 0, h // G, slots, :]
            V = kvf[pages, 1, h // G, slots, :]
            s = K @ qf[b, h] / np.sqrt(Dd)
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ V
    return out


def bf16_of(v):
    return np.array([oracle.f32_to_bf16(float(t)) for t in np.ravel(v)], np.uint16).reshape(np.shape(v))


def test_single_token_returns_v0_exactly():
    q, kv, bt, cl = make([1, 1, 1], seed=1)
    out = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    G = HQ // HKV
    for b in range(3):
        for h in range(HQ):
            np.testing.assert_array_equal(out[b, h], kv[bt[b, 0], 1, h // G, 0, :])


def test_constant_v_returns_v():
    q, kv, bt, cl = make([300, 777], seed=2)
    v = kv[0, 1, 0, 0, :].copy()
    kv[:, 1, :, :, :] = v
    out = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    for b in range(2):
        for h in range(HQ):
            np.testing.assert_array_equal(out[b, h], v)


def test_zero_query_gives_mean_of_v():
    q, kv, bt, cl = make([513], seed=3)
    q[:] = 0
    out = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    ref = numpy_reference(q, kv, bt, cl)
    check_close_bf16(out, bf16_of(ref), what="q=0")


@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 511, 512, 513, 600])
def test_within_tolerance_of_numpy_fp64(L):
    q, kv, bt, cl = make([L, max(1, L // 2)], seed=L)
    ref = numpy_reference(q, kv, bt, cl)
    exact = oracle.paged_decode_attn_exact(q, kv, bt, cl, HKV, PS)
    np.testing.assert_allclose(exact, ref, rtol=1e-10, atol=1e-12)
    out = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    check_close_bf16(out, bf16_of(ref), what=f"L={L}")


def test_swapped_k_and_v_would_fail():
    """Plant a mistake in a reference (K and V exchanged) and check the
    comparison above sees it."""
    q, kv, bt, cl = make([200], seed=4)
    swapped = kv[:, ::-1].copy()
    broken = numpy_reference(q, swapped, bt, cl)
    out = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    with pytest.raises(AssertionError):
        check_close_bf16(out, bf16_of(broken))


def test_zero_context_gives_zeros():
    q, kv, bt, cl = make([0, 40], seed=5)
    out = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    assert np.all(out[0] == 0)
    assert np.any(out[1] != 0)


def test_page_layout_invariance_and_no_leak():
    ctx = [1, 17, 256, 300, 529]
    q, kv, bt, cl = make(ctx, seed=6, shuffle=False)
    base = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    for s in (1, 2):
        kv2, bt2 = synth.relayout_kv(kv, bt, cl, PS, seed=100 + s)   # unused slots are NaN
        out = oracle.paged_decode_attn(q, kv2, bt2, cl, HKV, PS)
        np.testing.assert_array_equal(out, base)


def test_batch_composition_invariance():
    ctx = [70, 513, 1, 260]
    q, kv, bt, cl = make(ctx, seed=7)
    full = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    for b in range(len(ctx)):
        alone = oracle.paged_decode_attn(q[b:b + 1], kv, bt[b:b + 1], cl[b:b + 1], HKV, PS)
        np.testing.assert_array_equal(alone[0], full[b])
    perm = [2, 0, 3, 1]
    shuffled = oracle.paged_decode_attn(q[perm], kv, bt[perm], cl[perm], HKV, PS)
    np.testing.assert_array_equal(shuffled, full[perm])


def test_gqa_group_shares_kv_head():
    q, kv, bt, cl = make([333], seed=8)
    G = HQ // HKV
    for hk in range(HKV):
        q[0, hk * G:(hk + 1) * G] = q[0, hk * G]
    out = oracle.paged_decode_attn(q, kv, bt, cl, HKV, PS)
    for hk in range(HKV):
        for j in range(1, G):
            np.testing.assert_array_equal(out[0, hk * G + j], out[0, hk * G])
