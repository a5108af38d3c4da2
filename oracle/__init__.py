"""CPU oracle for the batch-invariant forward path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and
this package imports nothing from the product: it wraps ``bi_oracle.c``
(plain C, built with gcc) through ctypes and works on host numpy arrays of raw
bf16 bits (``uint16``).

Each wrapper names the schedule it follows; the C file cites the passages.
Functions ending in ``_exact`` are the fp64 definitions used to pin the
schedule oracle.  Parity status per function:

* ``gemm``           pinned (bf16-exact ordering cases, permutation and small
                     integer inputs, fp64 bound, row independence); the order
                     inside one 32-deep matrix-core block is a model and is
                     unpinned at that level (covered by the tolerance).
* ``rmsnorm``        pinned (fp64 bound, zero and +-1 rows, row independence).
* ``paged_decode_attn`` pinned (fp64 bound, one-token, constant-V and q=0
                     cases, page-layout invariance); the last bits of exp and
                     the association inside each 32-dim block of q.k are
                     unpinned (covered by the tolerance).
* ``philox4x64``     pinned against numpy's Philox bit generator.
* ``sample``         pinned (greedy = argmax with first-index ties, uniform
                     range and moments, Gumbel-max frequencies against the
                     softmax, temperature limits); its logarithms are the
                     platform's, so near-ties are unpinned.
* ``verify_commit``  pinned by worked cases of the commit-or-rollback rule.
* ``decoder.OracleDecoder`` (the stacked forward) pinned: reductions with
                     zeroed branches, row independence, the first token's
                     self-attention, and the whole composition (MLP active,
                     positions over several pages, a cache read by a later
                     call) against an independent float64 forward under
                     bounds that planted mistakes break.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRCS = [os.path.join(_HERE, "bi_oracle.c"), os.path.join(_HERE, "bi_oracle_layer.c"),
         os.path.join(_HERE, "bi_oracle_sample.c")]
_LIB = os.path.join(_HERE, "libbi_oracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-Wall", "-Wextra"]

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle's C sources into oracle/libbi_oracle.so with gcc."""
    deps = _SRCS + [os.path.join(_HERE, "bi_oracle.h")]
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            os.path.getmtime(f) for f in deps):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            p = ctypes.c_void_p
            i64 = ctypes.c_int64
            ci = ctypes.c_int
            lib.or_f32_to_bf16.argtypes = [ctypes.c_float]
            lib.or_f32_to_bf16.restype = ctypes.c_uint16
            lib.or_fold_f32.argtypes = [p, i64]
            lib.or_fold_f32.restype = ctypes.c_float
            lib.or_gemm.argtypes = [p, p, p, p, i64, i64, i64]
            lib.or_gemm_exact.argtypes = [p, p, p, i64, i64, i64]
            lib.or_gemm_absdot.argtypes = [p, p, p, i64, i64, i64]
            lib.or_rmsnorm.argtypes = [p, p, p, p, i64, i64, ctypes.c_float]
            lib.or_rmsnorm_exact.argtypes = [p, p, p, i64, i64, ctypes.c_double]
            lib.or_paged_decode_attn.argtypes = [p, p, p, p, p, i64, ci, ci, ci, ci, i64,
                                                 ctypes.c_float]
            lib.or_paged_decode_attn_exact.argtypes = [p, p, p, p, p, i64, ci, ci, ci, ci,
                                                       i64, ctypes.c_double]
            lib.or_rope_table.argtypes = [ctypes.c_double, ci, i64, p, p]
            lib.or_rope.argtypes = [p, p, p, i64, ci, ci, i64, p, p, i64]
            lib.or_silu_mul.argtypes = [p, p, i64, i64]
            lib.or_add.argtypes = [p, p, p, i64]
            lib.or_philox4x64.argtypes = [p, p, p]
            lib.or_philox4x64.restype = None
            lib.or_sample_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64, i64]
            lib.or_sample_uniform.restype = ctypes.c_float
            lib.or_sample.argtypes = [p, i64, i64, p, p, p, p, p, p]
            for f in ("or_gemm", "or_gemm_exact", "or_gemm_absdot", "or_rmsnorm",
                      "or_rmsnorm_exact", "or_paged_decode_attn",
                      "or_paged_decode_attn_exact", "or_rope_table", "or_rope",
                      "or_silu_mul", "or_add", "or_sample"):
                getattr(lib, f).restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected raw bf16 bits as uint16, got {a.dtype}")
    return a


def _check(rc: int, name: str):
    if rc != 0:
        raise RuntimeError(f"oracle {name} failed with code {rc}")


def f32_to_bf16(v: float) -> int:
    """Round one fp32 value to bf16 bits (nearest, ties to even)."""
    return int(_load().or_f32_to_bf16(ctypes.c_float(v)))


def fold_f32(values) -> float:
    """Left fold ((v0 + v1) + v2) + ... in fp32."""
    v = np.ascontiguousarray(values, dtype=np.float32)
    return float(_load().or_fold_f32(_ptr(v), v.size))


def gemm(x, w, return_f32: bool = False):
    """y = x @ w under the fixed segment schedule; x [M,K], w [K,N] bf16 bits."""
    x = _u16(x)
    w = _u16(w)
    M, K = x.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    y = np.empty((M, N), np.uint16)
    y32 = np.empty((M, N), np.float32)
    _check(_load().or_gemm(_ptr(x), _ptr(w), _ptr(y), _ptr(y32), M, N, K), "gemm")
    return (y, y32) if return_f32 else y


def gemm_exact(x, w) -> np.ndarray:
    x = _u16(x)
    w = _u16(w)
    M, K = x.shape
    N = w.shape[1]
    y = np.empty((M, N), np.float64)
    _check(_load().or_gemm_exact(_ptr(x), _ptr(w), _ptr(y), M, N, K), "gemm_exact")
    return y


def gemm_absdot(x, w) -> np.ndarray:
    x = _u16(x)
    w = _u16(w)
    M, K = x.shape
    N = w.shape[1]
    a = np.empty((M, N), np.float64)
    _check(_load().or_gemm_absdot(_ptr(x), _ptr(w), _ptr(a), M, N, K), "gemm_absdot")
    return a


def rmsnorm(x, g, eps: float = 1e-5, return_rinv: bool = False):
    """y = (x * r) * g with r = 1/sqrt(mean(x^2) + eps) under the fixed tree."""
    x = _u16(x)
    g = _u16(g)
    M, H = x.shape
    if g.shape != (H,):
        raise ValueError("gain must have shape [H]")
    y = np.empty((M, H), np.uint16)
    r = np.empty((M,), np.float32)
    _check(_load().or_rmsnorm(_ptr(x), _ptr(g), _ptr(y), _ptr(r), M, H,
                              ctypes.c_float(eps)), "rmsnorm")
    return (y, r) if return_rinv else y


def rmsnorm_exact(x, g, eps: float = 1e-5) -> np.ndarray:
    x = _u16(x)
    g = _u16(g)
    M, H = x.shape
    y = np.empty((M, H), np.float64)
    _check(_load().or_rmsnorm_exact(_ptr(x), _ptr(g), _ptr(y), M, H, eps), "rmsnorm_exact")
    return y


def _attn_args(q, kv, block_table, ctx_lens, num_kv_heads, page_size):
    q = _u16(q)
    kv = _u16(kv)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    cl = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, Hq, D = q.shape
    P = kv.shape[0]
    if kv.shape != (P, 2, num_kv_heads, page_size, D):
        raise ValueError("kv_pages must be [P, 2, Hkv, page_size, D]")
    if bt.ndim != 2 or bt.shape[0] != B or cl.shape != (B,):
        raise ValueError("block_table must be [B, max_blocks] and ctx_lens [B]")
    need = int(np.max((cl.astype(np.int64) + page_size - 1) // page_size, initial=0))
    if need > bt.shape[1]:
        raise ValueError("block_table too narrow for ctx_lens")
    for b in range(B):
        nb = (int(cl[b]) + page_size - 1) // page_size
        if nb > 0 and (bt[b, :nb].min() < 0 or bt[b, :nb].max() >= P):
            raise ValueError("block_table entry out of range")
    return q, kv, bt, cl, B, Hq, D


def paged_decode_attn(q, kv, block_table, ctx_lens, num_kv_heads: int = 8,
                      page_size: int = 16, scale: float | None = None) -> np.ndarray:
    """Decode attention under the fixed chunk/tile schedule (bf16 bits out)."""
    q, kv, bt, cl, B, Hq, D = _attn_args(q, kv, block_table, ctx_lens, num_kv_heads, page_size)
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    out = np.empty((B, Hq, D), np.uint16)
    _check(_load().or_paged_decode_attn(_ptr(q), _ptr(kv), _ptr(bt), _ptr(cl), _ptr(out), B,
                                        Hq, num_kv_heads, D, page_size, bt.shape[1],
                                        ctypes.c_float(scale)), "paged_decode_attn")
    return out


def paged_decode_attn_exact(q, kv, block_table, ctx_lens, num_kv_heads: int = 8,
                            page_size: int = 16, scale: float | None = None) -> np.ndarray:
    q, kv, bt, cl, B, Hq, D = _attn_args(q, kv, block_table, ctx_lens, num_kv_heads, page_size)
    if scale is None:
        scale = 1.0 / np.sqrt(float(D))
    out = np.empty((B, Hq, D), np.float64)
    _check(_load().or_paged_decode_attn_exact(_ptr(q), _ptr(kv), _ptr(bt), _ptr(cl), _ptr(out),
                                              B, Hq, num_kv_heads, D, page_size, bt.shape[1],
                                              scale), "paged_decode_attn_exact")
    return out


# ---------------------------------------------------------------------------
# Element-wise steps of the decoder layer (bi_oracle_layer.c)
# ---------------------------------------------------------------------------

def rope_table(theta: float, D: int, max_pos: int):
    """cos, sin as float32 [max_pos, D/2]: angle p * theta^(-2i/D) in double,
    each rounded once to fp32."""
    c = np.empty((max_pos, D // 2), dtype=np.float32)
    s = np.empty((max_pos, D // 2), dtype=np.float32)
    _check(_load().or_rope_table(ctypes.c_double(theta), D, max_pos, _ptr(c), _ptr(s)),
           "rope_table")
    return c, s


def rope(x, pos, heads: int, D: int, cos_t, sin_t):
    """Rotate-half RoPE of the first heads*D values of every row of x (bf16
    bits [M, >= heads*D]); returns [M, heads, D] bits."""
    x = _u16(x)
    M = x.shape[0]
    stride = int(np.prod(x.shape[1:])) if x.ndim > 1 else 0
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    c = np.ascontiguousarray(cos_t, dtype=np.float32)
    s = np.ascontiguousarray(sin_t, dtype=np.float32)
    y = np.empty((M, heads, D), dtype=np.uint16)
    _check(_load().or_rope(_ptr(x), _ptr(y), _ptr(pos), M, heads, D, stride, _ptr(c), _ptr(s),
                           c.shape[0]), "rope")
    return y


def silu_mul(gu):
    """bf16(silu(gate) * up) for gu = [gate | up] bf16 bits [M, 2F]."""
    gu = _u16(gu)
    M, F2 = gu.shape
    y = np.empty((M, F2 // 2), dtype=np.uint16)
    _check(_load().or_silu_mul(_ptr(gu), _ptr(y), M, F2 // 2), "silu_mul")
    return y


def add(a, b):
    """bf16(a + b) element-wise, one fp32 addition."""
    a, b = _u16(a), _u16(b)
    if a.shape != b.shape:
        raise ValueError("shapes differ")
    y = np.empty_like(a)
    _check(_load().or_add(_ptr(a), _ptr(b), _ptr(y), a.size), "add")
    return y


def philox4x64(counter, key):
    """Philox4x64-10 of one 4-word counter under a 2-word key (uint64)."""
    c = np.ascontiguousarray(counter, dtype=np.uint64)
    k = np.ascontiguousarray(key, dtype=np.uint64)
    out = np.empty(4, dtype=np.uint64)
    _load().or_philox4x64(_ptr(c), _ptr(k), _ptr(out))
    return out


def sample_uniform(seed: int, step: int, v: int) -> float:
    """The fp32 uniform that vocabulary entry v draws at (seed, step)."""
    return float(_load().or_sample_uniform(ctypes.c_uint64(seed), ctypes.c_uint64(step), v))


def sample(logits, seeds, steps, temps, return_scores: bool = False):
    """Per-row token: Gumbel-max over logits / T with Philox noise keyed by
    (seed, step), or argmax where T <= 0; ties to the first index."""
    logits = _u16(logits)
    M, V = logits.shape
    seeds = np.ascontiguousarray(seeds, dtype=np.uint64)
    steps = np.ascontiguousarray(steps, dtype=np.uint64)
    temps = np.ascontiguousarray(temps, dtype=np.float32)
    tok = np.empty(M, dtype=np.int32)
    best = np.empty(M, dtype=np.float32)
    second = np.empty(M, dtype=np.float32)
    _check(_load().or_sample(_ptr(logits), M, V, _ptr(seeds), _ptr(steps), _ptr(temps),
                             _ptr(tok), _ptr(best), _ptr(second)), "sample")
    return (tok, best, second) if return_scores else tok


def verify_commit(candidates, verified, row_start, commit_len):
    """Commit-or-rollback of grouped verification windows (LLM-42 digest,
    method): request r's window is rows row_start[r] .. row_start[r+1]-1 in
    position order; candidates[i] is the fast path's token for the position
    after row i, verified[i] the fixed-shape recompute's token there.  The
    leading matches are committed; at the first mismatch the recompute's
    token is committed instead and every later candidate is dropped.
    Returns (accepted, new commit length, correction token or -1)."""
    rs = [int(v) for v in row_start]
    acc, new_len, fix = [], [], []
    for r in range(len(rs) - 1):
        a, w = 0, rs[r + 1] - rs[r]
        while a < w and int(candidates[rs[r] + a]) == int(verified[rs[r] + a]):
            a += 1
        acc.append(a)
        if a < w:
            new_len.append(int(commit_len[r]) + a + 1)
            fix.append(int(verified[rs[r] + a]))
        else:
            new_len.append(int(commit_len[r]) + w)
            fix.append(-1)
    return (np.array(acc, np.int32), np.array(new_len, np.int32), np.array(fix, np.int32))
