"""Oracle of the decoder forward (test infrastructure only).

The same sequence of steps as a Llama-style decoder layer stack, each step
one of the oracle's own functions (GEMM, RMSNorm and paged attention from
bi_oracle.c; RoPE, the SiLU product and the residual add from
bi_oracle_layer.c); the embedding lookup and the KV-cache writes are plain
numpy indexing.  Rows are (request, position, token); each attends to its
request's cache up to and including its own position, and every row's KV is
written before any row attends (LLM-42 digest: grouped verification of the
tokens of several requests in one pass).  All values are raw bf16 bits.
"""
from __future__ import annotations

import numpy as np

from . import add, gemm, paged_decode_attn, rmsnorm, rope, rope_table, silu_mul


class OracleDecoder:
    def __init__(self, cfg, weight_bits: dict, num_pages: int, max_pos: int):
        self.cfg, self.w = cfg, weight_bits
        self.kv = [np.zeros((num_pages, 2, cfg.kv_heads, cfg.page_size, cfg.head_dim),
                            dtype=np.uint16) for _ in range(cfg.layers)]
        self.cos, self.sin = rope_table(cfg.theta, cfg.head_dim, max_pos)

    def forward(self, tokens, positions, block_table) -> np.ndarray:
        cfg, w = self.cfg, self.w
        tokens = np.asarray(tokens, dtype=np.int64)
        pos = np.asarray(positions, dtype=np.int32)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        M, D, PS = len(tokens), cfg.head_dim, cfg.page_size
        qd, kd = cfg.q_heads * D, cfg.kv_heads * D
        h = np.ascontiguousarray(w["embed"][tokens])
        for l in range(cfg.layers):
            x = rmsnorm(h, w[f"{l}.attn_norm"], cfg.eps)
            qkv = gemm(x, w[f"{l}.wqkv"])
            q = rope(np.ascontiguousarray(qkv[:, :qd]), pos, cfg.q_heads, D, self.cos, self.sin)
            k = rope(np.ascontiguousarray(qkv[:, qd:qd + kd]), pos, cfg.kv_heads, D,
                     self.cos, self.sin)
            v = qkv[:, qd + kd:].reshape(M, cfg.kv_heads, D)
            cache = self.kv[l]
            self.write_kv(cache, bt, pos, k, v)
            att = paged_decode_attn(q, cache, bt, pos + 1, num_kv_heads=cfg.kv_heads,
                                    page_size=PS)
            h = add(h, gemm(att.reshape(M, qd), w[f"{l}.wo"]))
            x = rmsnorm(h, w[f"{l}.ffn_norm"], cfg.eps)
            h = add(h, gemm(silu_mul(gemm(x, w[f"{l}.wgu"])), w[f"{l}.wdown"]))
        return gemm(rmsnorm(h, w["final_norm"], cfg.eps), w["lm_head"])

    def write_kv(self, cache, bt, pos, k, v):
        """Row m's key and value heads go to slot pos % page_size of page
        block_table[m][pos / page_size] (the paged layout the attention
        reads: token t of a request sits in page t / page_size, slot
        t % page_size)."""
        PS = self.cfg.page_size
        for m in range(len(pos)):
            page = bt[m, pos[m] // PS]
            cache[page, 0, :, pos[m] % PS, :] = k[m]
            cache[page, 1, :, pos[m] % PS, :] = v[m]
