"""bi_paged_prefill_attn on the GPU: many query rows of the same requests in
one call.  Every row's output is bitwise the decode entry point's for that
row (query-length invariance: a prompt token's attention output does not
depend on whether it was computed in a prefill of the whole prompt, a chunk
of it, or one token at a time), and within tolerance of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from invariant_bi_gemm_02_amd import synth
from tolerance import check_close_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
PS = synth.ATTN_PS


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def rows_for(req_lens, counts, seed, causal=True):
    """Row -> request ids, ctx lengths and row_start for `counts[r]` rows of
    request r.  Causal rows are the last counts[r] positions of the request
    (ctx = position + 1); otherwise ctx is drawn in [0, L_r]."""
    rng = np.random.default_rng(seed)
    rid, ctx = [], []
    for r, (L, n) in enumerate(zip(req_lens, counts)):
        if causal:
            c = np.arange(L - n + 1, L + 1)
        else:
            c = rng.integers(0, L + 1, n)
        rid += [r] * n
        ctx += list(c)
    row_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return np.array(rid, np.int64), np.array(ctx, np.int32), row_start


def both(gpu, q, kv, bt, rid, ctx, row_start, max_rows=None):
    qd, kvd = synth.from_bits(q, DEV), synth.from_bits(kv, DEV)
    mc = int(max(1, ctx.max()))
    pre = gpu.paged_prefill_attn(qd, kvd, t(bt), t(row_start), t(ctx), max_rows,
                                 max_ctx_len=mc)
    dec = gpu.paged_decode_attn(qd, kvd, t(bt[rid]), t(ctx), max_ctx_len=mc)
    torch.cuda.synchronize()
    return synth.to_bits(pre), synth.to_bits(dec)


@pytest.mark.parametrize("hkv", [32, 16, 8, 4])
def test_prefill_rows_equal_decode_rows(gpu, hkv):
    """Groups of 1, 2, 4 and 8 q heads per kv head; requests with 1, 3, 17,
    40 rows (one and several row blocks, ragged) and contexts across chunk
    and tile edges."""
    req_lens = np.array([1, 300, 17, 600], np.int32)
    counts = [1, 3, 17, 40]
    rid, ctx, row_start = rows_for(req_lens, counts, seed=hkv)
    q, kv, bt, _ = synth.attn_inputs(req_lens, seed=hkv, Hq=32, Hkv=hkv)
    qb = synth.bf16_normal((len(rid), 32, 128), seed=hkv + 50)
    pre, dec = both(gpu, synth.to_bits(qb), synth.to_bits(kv), bt, rid, ctx, row_start)
    np.testing.assert_array_equal(pre, dec)


def test_llama_shape_prompts_equal_decode_and_oracle(gpu):
    """Hq 32 / Hkv 8: six prompts of 1..1100 tokens prefilled in one call
    (every row causal), against decode per row (bitwise) and the oracle on a
    sample of rows."""
    req_lens = np.array([1, 64, 257, 511, 1100, 33], np.int32)
    rid, ctx, row_start = rows_for(req_lens, req_lens, seed=3)
    _, kv, bt, _ = synth.attn_inputs(req_lens, seed=3)
    q = synth.to_bits(synth.bf16_normal((len(rid), 32, 128), seed=4))
    kvb = synth.to_bits(kv)
    pre, dec = both(gpu, q, kvb, bt, rid, ctx, row_start)
    np.testing.assert_array_equal(pre, dec)
    sample = np.random.default_rng(5).choice(len(rid), 24, replace=False)
    sample = np.concatenate([sample, row_start[1:] - 1])      # every request's last row
    want = oracle.paged_decode_attn(np.ascontiguousarray(q[sample]), kvb,
                                    np.ascontiguousarray(bt[rid[sample]]), ctx[sample],
                                    synth.ATTN_HKV, PS)
    check_close_bf16(pre[sample], want, what="prefill vs oracle")


def test_non_causal_lengths_and_empty_rows(gpu):
    """Arbitrary per-row lengths, including 0 (zeros) and the request's full
    length; a request with no rows; rows past the one that needs most chunks."""
    req_lens = np.array([700, 5, 40, 1], np.int32)
    counts = [20, 0, 9, 2]
    rid, ctx, row_start = rows_for(req_lens, counts, seed=6, causal=False)
    ctx[0], ctx[3] = 0, 700
    _, kv, bt, _ = synth.attn_inputs(req_lens, seed=6)
    q = synth.to_bits(synth.bf16_normal((len(rid), 32, 128), seed=7))
    pre, dec = both(gpu, q, synth.to_bits(kv), bt, rid, ctx, row_start)
    np.testing.assert_array_equal(pre, dec)
    assert not pre[0].any()


def test_chunked_prefill_equals_one_pass(gpu):
    """The same prompt rows in one call, in chunks of 37 rows, and one row
    per call give the same bits (the decode entry point is the one-row case)."""
    req_lens = np.array([400, 150], np.int32)
    rid, ctx, row_start = rows_for(req_lens, req_lens, seed=8)
    _, kv, bt, _ = synth.attn_inputs(req_lens, seed=8)
    qd = synth.bf16_normal((len(rid), 32, 128), seed=9, device=DEV)
    kvd = kv.to(DEV)
    whole = synth.to_bits(gpu.paged_prefill_attn(qd, kvd, t(bt), t(row_start), t(ctx)))
    parts = []
    for s in range(0, len(rid), 37):
        e = min(len(rid), s + 37)
        reqs = np.unique(rid[s:e])
        rs = np.concatenate([[0], np.cumsum([(rid[s:e] == r).sum() for r in reqs])])
        parts.append(synth.to_bits(gpu.paged_prefill_attn(
            qd[s:e].contiguous(), kvd, t(bt[reqs]), t(rs.astype(np.int32)), t(ctx[s:e]),
            max_ctx_len=int(ctx.max()))))
    np.testing.assert_array_equal(np.concatenate(parts), whole)
    for m in (0, 255, 256, 399, 400, 549):
        one = gpu.paged_decode_attn(qd[m:m + 1].contiguous(), kvd, t(bt[rid[m:m + 1]]),
                                    t(ctx[m:m + 1]), max_ctx_len=int(ctx.max()))
        np.testing.assert_array_equal(synth.to_bits(one)[0], whole[m])


def test_row_start_past_the_rows_is_clamped(gpu):
    """row_start entries beyond the rows are clamped by the kernel: the rows
    that exist still get their decode result."""
    req_lens = np.array([90], np.int32)
    rid, ctx, _ = rows_for(req_lens, [10], seed=10)
    _, kv, bt, _ = synth.attn_inputs(req_lens, seed=10)
    q = synth.to_bits(synth.bf16_normal((10, 32, 128), seed=11))
    pre, dec = both(gpu, q, synth.to_bits(kv), bt, rid, ctx, np.array([0, 60], np.int32),
                    max_rows=10)
    np.testing.assert_array_equal(pre, dec)
