"""bi_paged_decode_attn on the GPU: parity with the oracle, and bitwise
invariance across batch composition, page layout and grid size."""
import numpy as np
import pytest
import torch

import oracle
from invariant_bi_gemm_02_amd import synth
from tolerance import check_close_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
HKV, PS = synth.ATTN_HKV, synth.ATTN_PS


def run(gpu, q, kv, bt, cl, max_ctx=None, fast=False):
    fn = gpu.paged_decode_attn_fast if fast else gpu.paged_decode_attn
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    mc = int(max(1, cl.max())) if max_ctx is None else max_ctx
    out = fn(q if torch.is_tensor(q) else synth.from_bits(q, DEV),
             kv if torch.is_tensor(kv) else synth.from_bits(kv, DEV), t(bt), t(cl), max_ctx_len=mc)
    torch.cuda.synchronize()
    return synth.to_bits(out)


@pytest.mark.parametrize("ctx", [[1], [15, 16, 17], [255, 256, 257], [63, 64, 65, 511, 513],
                                 [1000, 3, 2049]])
def test_edge_lengths_vs_oracle(gpu, ctx):
    ctx = np.array(ctx, np.int32)
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=int(ctx.sum()))
    qb, kvb = synth.to_bits(q), synth.to_bits(kv)
    got = run(gpu, qb, kvb, bt, cl)
    want = oracle.paged_decode_attn(qb, kvb, bt, cl, HKV, PS)
    stats = check_close_bf16(got, want, what=f"ctx={ctx.tolist()}")
    assert stats["bit_equal_share"] > 0.9


def test_single_token_is_v0_exactly(gpu):
    ctx = np.array([1, 1], np.int32)
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=11)
    kvb = synth.to_bits(kv)
    got = run(gpu, synth.to_bits(q), kvb, bt, cl)
    G = synth.ATTN_HQ // HKV
    for b in range(2):
        for h in range(synth.ATTN_HQ):
            np.testing.assert_array_equal(got[b, h], kvb[bt[b, 0], 1, h // G, 0])


def test_zero_context_gives_zeros(gpu):
    ctx = np.array([0, 77], np.int32)
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=12)
    bt[0, :] = 0
    got = run(gpu, synth.to_bits(q), synth.to_bits(kv), bt, cl)
    assert np.all(got[0] == 0) and np.any(got[1] != 0)


def test_config4_batch_layout_and_grid_invariance(gpu):
    """Llama-3-8B decode shape (32 q heads, 8 kv heads, dim 128, page 16),
    context lengths uniform in [512, 32768], shuffled pages.  Each request
    alone, in the batch, in a permuted batch, under a fresh page placement
    with NaN in every unused slot, and with a larger max_ctx_len: all
    bitwise equal."""
    B = 16
    ctx = synth.ctx_lens_uniform(B, seed=13)
    max_blocks = (32768 + 256) // PS   # room for the larger max_ctx_len below
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=13, max_blocks=max_blocks)
    qb, kvb = synth.to_bits(q), synth.to_bits(kv)
    kvd = synth.from_bits(kvb, DEV)
    full = run(gpu, qb, kvd, bt, cl)
    for b in (0, 5, B - 1):
        alone = run(gpu, qb[b:b + 1], kvd, bt[b:b + 1], cl[b:b + 1])
        np.testing.assert_array_equal(alone[0], full[b])
    perm = np.random.default_rng(0).permutation(B)
    np.testing.assert_array_equal(run(gpu, qb[perm], kvd, bt[perm], cl[perm]), full[perm])
    kv2, bt2 = synth.relayout_kv(kvb, bt, cl, PS, seed=99)
    np.testing.assert_array_equal(run(gpu, qb, kv2, bt2, cl), full)
    np.testing.assert_array_equal(run(gpu, qb, kvd, bt, cl, max_ctx=32768 + 256), full)
    for b in (0, 7):
        want = oracle.paged_decode_attn(qb[b:b + 1], kvb, bt[b:b + 1], cl[b:b + 1], HKV, PS)
        check_close_bf16(full[b:b + 1], want, what=f"request {b} L={cl[b]}")


def test_config4_b64_invariance_and_sampled_oracle(gpu):
    """The largest batch of the workload: B = 64, context lengths uniform in
    [512, 32768], shuffled pages.  Requests alone and in a permuted batch are
    bitwise equal to the batch run; 16 sampled requests agree with the
    oracle."""
    B = 64
    ctx = synth.ctx_lens_uniform(B, seed=41)
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=41)
    qb, kvb = synth.to_bits(q), synth.to_bits(kv)
    kvd = synth.from_bits(kvb, DEV)
    full = run(gpu, qb, kvd, bt, cl)
    for b in (0, 17, 40, B - 1):
        alone = run(gpu, qb[b:b + 1], kvd, bt[b:b + 1], cl[b:b + 1])
        np.testing.assert_array_equal(alone[0], full[b])
    perm = np.random.default_rng(1).permutation(B)
    np.testing.assert_array_equal(run(gpu, qb[perm], kvd, bt[perm], cl[perm]), full[perm])
    for b in range(0, B, 4):
        want = oracle.paged_decode_attn(qb[b:b + 1], kvb, bt[b:b + 1], cl[b:b + 1], HKV, PS)
        check_close_bf16(full[b:b + 1], want, what=f"request {b} L={cl[b]}")


@pytest.mark.parametrize("B", [1, 4, 64])
def test_fast_twin_parity(gpu, B):
    ctx = synth.ctx_lens_uniform(B, seed=20 + B, lo=512, hi=8192)
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=20 + B)
    qb, kvb = synth.to_bits(q), synth.to_bits(kv)
    got = run(gpu, qb, kvb, bt, cl, fast=True)
    for b in sorted(set([0, B - 1])):
        want = oracle.paged_decode_attn(qb[b:b + 1], kvb, bt[b:b + 1], cl[b:b + 1], HKV, PS)
        check_close_bf16(got[b:b + 1], want, what=f"fast B={B} b={b}")


def test_default_scale_through_the_c_abi(gpu):
    """A descriptor scale <= 0 (or -0) selects 1/sqrt(head_dim), computed in
    the library: the same bits as passing fp32(1/sqrt(128)) explicitly, and
    within tolerance of the oracle's default."""
    import ctypes
    from invariant_bi_gemm_02_amd import _lib
    lib = gpu.load()
    ctx = np.array([300, 17, 1024], np.int32)
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=77)
    qd, kvd = q.to(DEV), kv.to(DEV)
    btd = torch.from_numpy(bt).to(DEV)
    cld = torch.from_numpy(cl).to(DEV)
    B = len(ctx)
    outs = []
    explicit = float(np.float32(1.0) / np.sqrt(np.float32(128)))
    for scale in (0.0, -0.0, -1.0, explicit):
        d = _lib.AttnDesc(B, 32, HKV, 128, PS, bt.shape[1], kv.shape[0], int(ctx.max()), scale)
        need = lib.bi_attn_workspace_bytes(ctypes.byref(d))
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        out = torch.empty_like(qd)
        st = lib.bi_paged_decode_attn(qd.data_ptr(), kvd.data_ptr(), btd.data_ptr(),
                                      cld.data_ptr(), out.data_ptr(), ctypes.byref(d),
                                      ws.data_ptr(), need, None)
        assert st == 0
        torch.cuda.synchronize()
        outs.append(synth.to_bits(out))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    want = oracle.paged_decode_attn(synth.to_bits(q), synth.to_bits(kv), bt, cl, HKV, PS)
    check_close_bf16(outs[0], want, what="default scale")


def test_longest_supported_context(gpu):
    """A request at the largest context the entry point takes (262144
    tokens: 1024 chunks, a 1 GiB page pool): within tolerance of the oracle,
    and bitwise the same alone as beside a one-token request with a
    max_ctx_len that sizes the grid for both."""
    L = 262144
    ctx = np.array([L, 1], np.int32)
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=91)
    qb, kvb = synth.to_bits(q), synth.to_bits(kv)
    kvd = kv.to(DEV)
    both = run(gpu, q.to(DEV), kvd, bt, cl, max_ctx=L)
    alone = run(gpu, q[:1].contiguous().to(DEV), kvd, bt[:1], cl[:1], max_ctx=L)
    np.testing.assert_array_equal(alone, both[:1])
    want = oracle.paged_decode_attn(qb[:1], kvb, bt[:1], cl[:1], HKV, PS)
    check_close_bf16(alone, want, what="262144-token context")
    # the one-token request reads its single value vector exactly
    page, slot = int(bt[1, 0]), 0
    for h in range(32):
        np.testing.assert_array_equal(both[1, h], kvb[page, 1, h // 4, slot])


@pytest.mark.parametrize("seed", range(6))
def test_random_groups_and_lengths_vs_oracle_and_alone(gpu, seed):
    """Seeded random cases over the group sizes the kernel has (G = 1, 2, 4,
    8 query heads per kv head), batch sizes 1-6 and context lengths 1-3000
    (tile and chunk boundaries included at random): within tolerance of the
    oracle, and every request alone bitwise equal to its row in the batch."""
    rng = np.random.default_rng(500 + seed)
    G = [1, 2, 4, 8, 2, 8][seed]
    hkv = [8, 4, 2, 1, 2, 4][seed]
    B = int(rng.integers(1, 7))
    ctx = rng.integers(1, 3001, size=B).astype(np.int32)
    ctx[rng.integers(0, B)] = [1, 64, 256, 257, 512, 2048][seed]
    q, kv, bt, cl = synth.attn_inputs(ctx, seed=600 + seed, Hq=G * hkv, Hkv=hkv)
    qb, kvb = synth.to_bits(q), synth.to_bits(kv)
    got = run(gpu, qb, kvb, bt, cl)
    want = oracle.paged_decode_attn(qb, kvb, bt, cl, hkv, PS)
    check_close_bf16(got, want, what=f"G={G} Hkv={hkv} ctx={ctx.tolist()}")
    for b in range(B):
        alone = run(gpu, qb[b:b + 1], kvb, bt[b:b + 1], cl[b:b + 1])
        np.testing.assert_array_equal(alone[0], got[b])
