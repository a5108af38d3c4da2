"""Seeded synthetic inputs for the batch-invariant forward path.

This module holds no arithmetic of the method itself: it only draws random
tensors and rounds them to bf16 (torch's round-to-nearest-even), so that the
HIP path and the CPU oracle consume the same bytes.  Shapes and distributions
follow the Llama-3-8B-shaped workloads the pages discuss (an 8B Llama served
in bf16): activations N(0,1), weights N(0,0.02), RMSNorm gain N(1,0.1), K/V
N(0,1), paged KV with a shuffled page pool and context lengths uniform in
[512, 32768].

Host arrays are numpy ``uint16`` holding raw bf16 bits; device tensors are
torch ``bfloat16``.
"""
from __future__ import annotations

import numpy as np
import torch

# Llama-3-8B linear shapes as (name, K, N): y[M,N] = x[M,K] . W[K,N]
LLAMA3_8B_LINEARS = (
    ("qkv", 4096, 6144),
    ("o", 4096, 4096),
    ("gate_up", 4096, 28672),
    ("down", 14336, 4096),
)

# Batch sizes swept for the linears: powers of two and their odd neighbours.
M_SWEEP = (1, 2, 3, 4, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129,
           255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2047, 2048)

RMSNORM_M = (1, 3, 8, 31, 64, 257, 512)

ATTN_HQ, ATTN_HKV, ATTN_D, ATTN_PS = 32, 8, 128, 16


def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def bf16_normal(shape, seed: int, mean: float = 0.0, std: float = 1.0,
                device="cpu") -> torch.Tensor:
    """A bf16 tensor drawn N(mean, std^2) from its own seeded generator."""
    g = _gen(seed, device)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(torch.bfloat16)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bits of a tensor as a host uint16 array."""
    if t.dtype != torch.bfloat16:
        raise TypeError("expected a bfloat16 tensor")
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    """bf16 tensor holding the given raw bits."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)


def gemm_inputs(M: int, K: int, N: int, seed: int, w_std: float = 0.02, x_std: float = 1.0,
                device="cpu"):
    """x[M,K] ~ N(0, x_std^2) and W[K,N] ~ N(0, w_std^2), both bf16."""
    x = bf16_normal((M, K), seed * 2 + 1, std=x_std, device=device)
    w = bf16_normal((K, N), seed * 2 + 2, std=w_std, device=device)
    return x, w


def rmsnorm_inputs(M: int, H: int, seed: int, device="cpu"):
    """x[M,H] ~ N(0,1), gain g[H] ~ N(1, 0.1^2)."""
    x = bf16_normal((M, H), seed * 2 + 1, device=device)
    g = bf16_normal((H,), seed * 2 + 2, mean=1.0, std=0.1, device=device)
    return x, g


def attn_layout(ctx_lens, page_size: int, seed: int, shuffle: bool = True,
                extra_pages: int = 0, max_blocks: int | None = None):
    """Page pool size and block table for the given context lengths.

    Each request gets ceil(L/page_size) pages from a pool of all pages
    (plus ``extra_pages`` unused ones); with ``shuffle`` the pool is a random
    permutation, otherwise pages are handed out in order.  Unused table
    entries are -1.
    """
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    nblk = (np.maximum(ctx, 0) + page_size - 1) // page_size
    total = int(nblk.sum()) + int(extra_pages)
    rng = np.random.default_rng(seed)
    pool = rng.permutation(total) if shuffle else np.arange(total)
    mb = int(nblk.max(initial=1)) if max_blocks is None else int(max_blocks)
    mb = max(mb, 1)
    bt = np.full((len(ctx), mb), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = pool[off:off + n]
        off += int(n)
    return max(total, 1), bt


def ctx_lens_uniform(B: int, seed: int, lo: int = 512, hi: int = 32768) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def attn_inputs(ctx_lens, seed: int, shuffle: bool = True, extra_pages: int = 0,
                max_blocks: int | None = None, Hq: int = ATTN_HQ, Hkv: int = ATTN_HKV,
                D: int = ATTN_D, page_size: int = ATTN_PS, device="cpu"):
    """q[B,Hq,D], kv_pages[P,2,Hkv,PS,D] (all N(0,1) bf16), block_table, ctx_lens."""
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    P, bt = attn_layout(ctx, page_size, seed * 3 + 1, shuffle, extra_pages, max_blocks)
    q = bf16_normal((len(ctx), Hq, D), seed * 3 + 2, device=device)
    kv = bf16_normal((P, 2, Hkv, page_size, D), seed * 3 + 3, device=device)
    return q, kv, bt, ctx


def relayout_kv(kv_bits: np.ndarray, bt: np.ndarray, ctx_lens, page_size: int, seed: int,
                fill_bits: int = 0x7FC0):
    """The same logical K/V under a fresh random page placement.

    Returns (kv2, bt2): every used page of every request is copied to a new
    slot of a freshly permuted pool; all other slots hold ``fill_bits``
    (default a quiet NaN) so that reading an unused slot shows in the output.
    """
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    nblk = (np.maximum(ctx, 0) + page_size - 1) // page_size
    total = int(nblk.sum())
    rng = np.random.default_rng(seed)
    P2 = total + 3
    pool = rng.permutation(P2)[:total]
    kv2 = np.full((P2,) + kv_bits.shape[1:], fill_bits, dtype=np.uint16)
    bt2 = np.full(bt.shape, -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        for j in range(int(n)):
            src = int(bt[b, j])
            dst = int(pool[off + j])
            bt2[b, j] = dst
            # copy only the valid slots of the last page; the rest keep the fill
            valid = min(page_size, int(ctx[b]) - j * page_size)
            kv2[dst, :, :, :valid, :] = kv_bits[src, :, :, :valid, :]
        off += int(n)
    return kv2, bt2


# ---------------------------------------------------------------------------
# Decoder (Llama-3-8B-shaped, random init) and LLM-42-style verify batches
# ---------------------------------------------------------------------------

class DecoderConfig:
    """Sizes of a Llama-style decoder (no arithmetic here)."""

    def __init__(self, layers=32, hidden=4096, q_heads=32, kv_heads=8, ffn=14336,
                 vocab=128256, theta=5e5, eps=1e-5, head_dim=128, page_size=16):
        self.layers, self.hidden, self.q_heads, self.kv_heads = layers, hidden, q_heads, kv_heads
        self.ffn, self.vocab, self.theta, self.eps = ffn, vocab, theta, eps
        self.head_dim, self.page_size = head_dim, page_size

    @property
    def qkv_width(self) -> int:
        return (self.q_heads + 2 * self.kv_heads) * self.head_dim


LLAMA3_8B = DecoderConfig()
# A small configuration with the same head shape, for oracle comparisons.
TINY = DecoderConfig(layers=2, hidden=512, q_heads=4, kv_heads=2, ffn=1024, vocab=1024)


def decoder_weights(cfg: DecoderConfig, seed: int, device="cpu") -> dict:
    """Random-init bf16 weights: matrices N(0, 0.02^2) laid out [in, out]
    (y = x W), gains N(1, 0.1^2), embedding N(0, 1)."""
    w = {"embed": bf16_normal((cfg.vocab, cfg.hidden), seed * 100 + 1, device=device)}
    for l in range(cfg.layers):
        b = seed * 100 + 10 + 8 * l
        w[f"{l}.attn_norm"] = bf16_normal((cfg.hidden,), b, mean=1.0, std=0.1, device=device)
        w[f"{l}.wqkv"] = bf16_normal((cfg.hidden, cfg.qkv_width), b + 1, std=0.02, device=device)
        w[f"{l}.wo"] = bf16_normal((cfg.q_heads * cfg.head_dim, cfg.hidden), b + 2, std=0.02,
                                   device=device)
        w[f"{l}.ffn_norm"] = bf16_normal((cfg.hidden,), b + 3, mean=1.0, std=0.1, device=device)
        w[f"{l}.wgu"] = bf16_normal((cfg.hidden, 2 * cfg.ffn), b + 4, std=0.02, device=device)
        w[f"{l}.wdown"] = bf16_normal((cfg.ffn, cfg.hidden), b + 5, std=0.02, device=device)
    w["final_norm"] = bf16_normal((cfg.hidden,), seed * 100 + 2, mean=1.0, std=0.1,
                                  device=device)
    w["lm_head"] = bf16_normal((cfg.hidden, cfg.vocab), seed * 100 + 3, std=0.02, device=device)
    return w


class Requests:
    """A set of requests sharing one page pool per layer: prompt tokens, and
    for each request a block table row with room for max_len tokens.  Pages
    are handed out from a shuffled pool."""

    def __init__(self, prompt_lens, max_len: int, vocab: int, page_size: int, seed: int):
        rng = np.random.default_rng(seed)
        self.prompt_lens = [int(x) for x in prompt_lens]
        self.max_blocks = -(-max_len // page_size)
        n = len(self.prompt_lens)
        self.num_pages = n * self.max_blocks
        perm = rng.permutation(self.num_pages).astype(np.int32)
        self.block_table = perm.reshape(n, self.max_blocks)
        self.prompts = [rng.integers(0, vocab, size=L).astype(np.int32) for L in self.prompt_lens]

    def rows(self, req_ids, positions, tokens):
        """Per-row arrays for a forward over (request, position, token) rows."""
        req_ids = np.asarray(req_ids, dtype=np.int64)
        return (np.asarray(tokens, dtype=np.int32), np.asarray(positions, dtype=np.int32),
                np.ascontiguousarray(self.block_table[req_ids]))


def grouped_rows(req: "Requests", segments):
    """Rows of a multi-query forward from segments [(request, positions,
    tokens)], each one request's run of rows: tokens [M], positions [M], the
    segments' block table rows [S, max_blocks] and row_start [S + 1]."""
    tok = np.concatenate([np.asarray(s[2], np.int32) for s in segments])
    pos = np.concatenate([np.asarray(s[1], np.int32) for s in segments])
    bt = np.ascontiguousarray(req.block_table[[s[0] for s in segments]])
    row_start = np.concatenate([[0], np.cumsum([len(s[1]) for s in segments])]).astype(np.int32)
    return tok, pos, bt, row_start


def verify_groups(n_requests: int, total: int, seed: int):
    """LLM-42-style grouped verification: split `total` window tokens over
    the requests (each gets at least one), in a shuffled row order."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, total), size=n_requests - 1, replace=False))
    sizes = np.diff(np.concatenate([[0], cuts, [total]]))
    return [int(s) for s in sizes]
