"""A Llama-style decoder forward assembled from the library's calls.

Orchestration only: every arithmetic step is one of the C-ABI calls (the
batch-invariant GEMM, RMSNorm (fused with the residual add before it) and
paged decode attention, and the element-wise embedding, RoPE, KV append and
SiLU product), run on torch's current stream; torch supplies buffers.  Each row of a forward is
one token of some request at some position, attending to its request's KV
cache up to and including itself, so a batch may mix any number of requests
and window lengths -- the LLM-42 digest's grouped verification, where the
tokens of several requests are checked in one fixed-shape pass.  Since every
call is row-independent, a row's logits are bit-identical whether it is run
alone, with the rest of its request, or grouped with other requests, and
whether its prompt was prefilled in one pass, in chunks or token by token.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as bi


class Decoder:
    def __init__(self, cfg, weights: dict, num_pages: int, max_pos: int, device="cuda"):
        if cfg.head_dim != 128 or cfg.page_size != 16:
            raise ValueError("the kernels take head_dim 128 and page size 16")
        self.cfg, self.w, self.device = cfg, weights, device
        shape = (num_pages, 2, cfg.kv_heads, cfg.page_size, cfg.head_dim)
        self.kv = [torch.zeros(shape, dtype=torch.bfloat16, device=device)
                   for _ in range(cfg.layers)]
        self.cos, self.sin = bi.rope_table(cfg.theta, cfg.head_dim, max_pos, device)
        self.max_pos = max_pos

    def prepare(self, tokens, positions, block_table, row_start=None):
        """Device copies of a forward's row arrays (host arrays in): tokens
        [M], positions [M], block_table [M, max_blocks] (the row's request).

        With row_start ([R + 1], host) the rows come grouped by request --
        rows row_start[r] .. row_start[r+1]-1 belong to request r, and
        block_table has one row per request ([R, max_blocks]) -- and the
        attention runs the multi-query entry point, which loads a request's
        K/V once for many rows and gives each row the same bits as the
        per-row path."""
        positions = np.asarray(positions, dtype=np.int32)
        if positions.min() < 0 or positions.max() >= self.max_pos:
            raise ValueError("position outside the rope table")
        dev = self.device
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        grouped = None
        if row_start is not None:
            row_start = np.asarray(row_start, dtype=np.int32)
            counts = np.diff(row_start)
            if row_start[0] != 0 or row_start[-1] != len(positions) or (counts < 0).any():
                raise ValueError("row_start must run from 0 to the number of rows")
            grouped = (up(block_table), up(row_start), int(counts.max()))
            block_table = np.repeat(np.asarray(block_table), counts, axis=0)
        # a row attends to its request's tokens up to and including itself
        return (up(tokens), up(positions), up(positions + 1), up(block_table),
                int(positions.max()) + 1, grouped)

    def run(self, rows, logit_rows=None) -> torch.Tensor:
        """Logits [M, vocab] (bf16) for rows from prepare(); with logit_rows
        (device int32 row indices) only those rows' logits, in that order
        (a prefill needs each prompt's last row only).  The normalized rows
        are gathered with the embedding kernel; every step is row-independent,
        so their bits are the same either way."""
        cfg, w = self.cfg, self.w
        tok, pos, ctx, bt, max_ctx, grouped = rows
        M = tok.shape[0]
        qd, kd = cfg.q_heads * cfg.head_dim, cfg.kv_heads * cfg.head_dim
        h = bi.embed(tok, w["embed"])
        x = bi.rmsnorm(h, w["0.attn_norm"], cfg.eps)
        for l in range(cfg.layers):
            qkv = bi.gemm(x, w[f"{l}.wqkv"])
            q = bi.rope(qkv[:, :qd], cfg.q_heads, pos, self.cos, self.sin)
            k = bi.rope(qkv[:, qd:qd + kd], cfg.kv_heads, pos, self.cos, self.sin)
            bi.kv_append(k.view(M, kd), qkv[:, qd + kd:], self.kv[l], bt, pos)
            if grouped is None:
                att = bi.paged_decode_attn(q, self.kv[l], bt, ctx, max_ctx_len=max_ctx)
            else:
                att = bi.paged_prefill_attn(q, self.kv[l], grouped[0], grouped[1], ctx,
                                            grouped[2], max_ctx_len=max_ctx)
            # each residual add and the norm after it in one call (the same
            # bits as bi.add then bi.rmsnorm); the sum replaces h in place
            h, x = bi.add_rmsnorm(h, bi.gemm(att.view(M, qd), w[f"{l}.wo"]),
                                  w[f"{l}.ffn_norm"], cfg.eps, sum_out=h)
            a = bi.silu_mul(bi.gemm(x, w[f"{l}.wgu"]))
            nxt = w[f"{l + 1}.attn_norm"] if l + 1 < cfg.layers else w["final_norm"]
            h, x = bi.add_rmsnorm(h, bi.gemm(a, w[f"{l}.wdown"]), nxt, cfg.eps, sum_out=h)
        if logit_rows is not None:
            x = bi.embed(logit_rows, x)
        return bi.gemm(x, w["lm_head"])

    def forward(self, tokens, positions, block_table, row_start=None) -> torch.Tensor:
        """prepare() then run(): logits [M, vocab] for host row arrays."""
        return self.run(self.prepare(tokens, positions, block_table, row_start))
