"""ctypes binding of libbi.so (argument marshalling only).

Tensors are torch device tensors; the library receives their raw device
pointers and torch's current HIP stream.  Nothing here computes: a missing
library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbi.so")

_STATUS = {0: "BI_OK", -1: "BI_ERR_NULL", -2: "BI_ERR_SHAPE", -3: "BI_ERR_UNSUPPORTED",
           -4: "BI_ERR_WORKSPACE", -5: "BI_ERR_HIP", -6: "BI_ERR_SCRATCH"}


class BiError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)} ({status})")


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("max_ctx_len", ctypes.c_int32),
                ("scale", ctypes.c_float)]


EXPORTS = ("bi_version", "bi_status_string", "bi_gemm_workspace_bytes", "bi_gemm",
           "bi_gemm_fast_workspace_bytes", "bi_gemm_fast", "bi_rmsnorm", "bi_rmsnorm_fast",
           "bi_attn_workspace_bytes", "bi_paged_decode_attn", "bi_attn_fast_workspace_bytes",
           "bi_paged_decode_attn_fast", "bi_embed", "bi_rope_table", "bi_rope", "bi_kv_append",
           "bi_silu_mul", "bi_add", "bi_paged_prefill_attn",
           "bi_gemm_segments", "bi_gemm_fold", "bi_sample", "bi_verify_commit",
           "bi_sample_workspace_bytes", "bi_add_rmsnorm", "bi_gemm_noalloc",
           "bi_ceiling_mfma", "bi_ceiling_read")

_lock = threading.Lock()
_lib = None


def load(path: str | None = None):
    """Load libbi.so once; raise if it was never built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(
                f"HIP library {p} is missing: build it first (python -c 'import __graft_entry__ as "
                f"g; g.build()'); there is no fallback path")
        lib = ctypes.CDLL(p)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        lib.bi_version.restype = ctypes.c_char_p
        lib.bi_version.argtypes = []
        lib.bi_status_string.restype = ctypes.c_char_p
        lib.bi_status_string.argtypes = [ctypes.c_int]
        for f in ("bi_gemm_workspace_bytes", "bi_gemm_fast_workspace_bytes"):
            getattr(lib, f).restype = sz
            getattr(lib, f).argtypes = [i64, i64, i64]
        for f in ("bi_gemm", "bi_gemm_fast"):
            getattr(lib, f).restype = ctypes.c_int
            getattr(lib, f).argtypes = [vp, vp, vp, i64, i64, i64, vp, sz, vp]
        for f in ("bi_rmsnorm", "bi_rmsnorm_fast"):
            getattr(lib, f).restype = ctypes.c_int
            getattr(lib, f).argtypes = [vp, vp, vp, i64, i64, ctypes.c_float, vp]
        lib.bi_add_rmsnorm.restype = ctypes.c_int
        lib.bi_add_rmsnorm.argtypes = [vp, vp, vp, vp, vp, i64, i64, ctypes.c_float, vp]
        for f in ("bi_attn_workspace_bytes", "bi_attn_fast_workspace_bytes"):
            getattr(lib, f).restype = sz
            getattr(lib, f).argtypes = [ctypes.POINTER(AttnDesc)]
        for f in ("bi_paged_decode_attn", "bi_paged_decode_attn_fast"):
            getattr(lib, f).restype = ctypes.c_int
            getattr(lib, f).argtypes = [vp, vp, vp, vp, vp, ctypes.POINTER(AttnDesc), vp, sz, vp]
        i32 = ctypes.c_int32
        sigs = {
            "bi_embed": [vp, vp, vp, i64, i64, i64, vp],
            "bi_rope_table": [ctypes.c_double, i32, i64, vp, vp],
            "bi_rope": [vp, i64, vp, vp, vp, vp, i64, i32, i32, i64, vp],
            "bi_kv_append": [vp, i64, vp, i64, vp, vp, vp, i64, i32, i32, i32, i32, i64, vp],
            "bi_silu_mul": [vp, vp, i64, i64, vp],
            "bi_add": [vp, vp, vp, i64, vp],
            "bi_paged_prefill_attn": [vp, vp, vp, vp, vp, vp, ctypes.POINTER(AttnDesc), i32, i32,
                                      vp, sz, vp],
            "bi_gemm_segments": [vp, vp, vp, i64, i64, i64, vp],
            "bi_sample": [vp, i64, i64, vp, vp, vp, vp, vp, sz, vp],
            "bi_sample_workspace_bytes": [i64],
            "bi_verify_commit": [vp, vp, i32, vp, i32, vp, vp, vp, vp],
            "bi_gemm_fold": [vp, vp, i64, i64, i64, vp],
            "bi_gemm_noalloc": [vp, vp, vp, i64, i64, i64, vp],
            "bi_ceiling_mfma": [vp, i64, i64, vp],
            "bi_ceiling_read": [vp, i64, vp, vp],
        }
        for f, a in sigs.items():
            getattr(lib, f).restype = ctypes.c_int
            getattr(lib, f).argtypes = a
        lib.bi_sample_workspace_bytes.restype = sz
        _lib = lib
        return lib


def version() -> str:
    return load().bi_version().decode()


class Workspace:
    """A device scratch buffer that grows on demand (one per stream).

    Under HIP graph capture every call gets a buffer of its own instead: the
    captured kernels keep its address for every replay, so it must belong to
    the graph's memory pool, which lives as long as the graph.  A cached
    buffer would not: a later, larger call frees it, and once its pool is
    released (torch empties the cache before each capture) the replays would
    write to unmapped memory."""

    def __init__(self, device=None):
        self.device = torch.device(device or "cuda")
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if torch.cuda.is_current_stream_capturing():
            return torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws: dict = {}


def _ws_for(device: torch.device, ws: Workspace | None) -> Workspace:
    if ws is not None:
        return ws
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    w = _default_ws.get(key)
    if w is None:
        w = _default_ws[key] = Workspace(device)
    return w


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check_bf16(t: torch.Tensor, name: str, ndim: int):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bfloat16 tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-D tensor")


def _raise(status: int, where: str):
    if status != 0:
        raise BiError(status, where)


def gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().bi_gemm_workspace_bytes(M, N, K))


def gemm_fast_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().bi_gemm_fast_workspace_bytes(M, N, K))


def _gemm(fn_name, wsq, x, w, out, ws):
    lib = load()
    _check_bf16(x, "x", 2)
    _check_bf16(w, "W", 2)
    M, K = x.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError(f"x is [M,{K}] but W is [{K2},N]")
    if x.device != w.device:
        raise ValueError("x and W on different devices")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _check_bf16(out, "out", 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    need = int(getattr(lib, wsq)(M, N, K))
    buf = _ws_for(x.device, ws).get(need)
    st = getattr(lib, fn_name)(x.data_ptr(), w.data_ptr(), out.data_ptr(), M, N, K,
                               buf.data_ptr(), buf.numel(), _stream(x.device))
    _raise(st, fn_name)
    return out


def ceiling_mfma(iters: int, workgroups: int, out=None, device=None):
    """Launch the matrix-core-only loop (a measurement helper); returns the
    per-lane output tensor and the flops one launch performs."""
    lib = load()
    dev = torch.device(device or "cuda")
    if out is None:
        out = torch.empty(workgroups * 256, dtype=torch.float32, device=dev)
    _raise(lib.bi_ceiling_mfma(out.data_ptr(), int(iters), int(workgroups), _stream(dev)),
           "bi_ceiling_mfma")
    return out, float(workgroups) * 4 * iters * 8 * 16384


CEILING_READ_OUT_WORDS = 8192


def ceiling_read(buf: torch.Tensor, out=None):
    """Stream every byte of the device tensor `buf` once (a measurement
    helper); returns the per-wave output words (int32 tensor of
    CEILING_READ_OUT_WORDS, allocated here when None)."""
    lib = load()
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise TypeError("buf must be a contiguous device tensor")
    if out is None:
        out = torch.empty(CEILING_READ_OUT_WORDS, dtype=torch.int32, device=buf.device)
    elif out.numel() < CEILING_READ_OUT_WORDS or out.element_size() != 4 or not out.is_cuda:
        raise ValueError("out must be a device tensor of CEILING_READ_OUT_WORDS 4-byte words")
    _raise(lib.bi_ceiling_read(buf.data_ptr(), buf.numel() * buf.element_size(), out.data_ptr(),
                               _stream(buf.device)), "bi_ceiling_read")
    return out


def gemm_noalloc(x, w, out=None):
    """y = x @ W through bi_gemm_noalloc: bi_gemm's bits, with the library's
    static scratch instead of a workspace (out is allocated here when None;
    pass it to allocate nothing)."""
    lib = load()
    _check_bf16(x, "x", 2)
    _check_bf16(w, "W", 2)
    M, K = x.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError(f"x is [M,{K}] but W is [{K2},N]")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    else:
        _check_bf16(out, "out", 2)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    st = lib.bi_gemm_noalloc(x.data_ptr(), w.data_ptr(), out.data_ptr(), M, N, K,
                             _stream(x.device))
    _raise(st, "bi_gemm_noalloc")
    return out


def gemm(x, w, out=None, ws: Workspace | None = None):
    """y = x @ W (batch-invariant).  x [M,K], W [K,N] bf16 device tensors."""
    return _gemm("bi_gemm", "bi_gemm_workspace_bytes", x, w, out, ws)


def gemm_fast(x, w, out=None, ws: Workspace | None = None):
    """y = x @ W with M-tuned tiles and split (not batch-invariant)."""
    return _gemm("bi_gemm_fast", "bi_gemm_fast_workspace_bytes", x, w, out, ws)


def _rmsnorm(fn_name, x, g, eps, out):
    lib = load()
    _check_bf16(x, "x", 2)
    _check_bf16(g, "g", 1)
    M, H = x.shape
    if g.shape[0] != H:
        raise ValueError("gain must have shape [H]")
    if out is None:
        out = torch.empty_like(x)
    else:
        _check_bf16(out, "out", 2)
        if tuple(out.shape) != (M, H):
            raise ValueError("out has the wrong shape")
    st = getattr(lib, fn_name)(x.data_ptr(), g.data_ptr(), out.data_ptr(), M, H,
                               ctypes.c_float(eps), _stream(x.device))
    _raise(st, fn_name)
    return out


def rmsnorm(x, g, eps: float = 1e-5, out=None):
    return _rmsnorm("bi_rmsnorm", x, g, eps, out)


def rmsnorm_fast(x, g, eps: float = 1e-5, out=None):
    return _rmsnorm("bi_rmsnorm_fast", x, g, eps, out)


def add_rmsnorm(a, b, g, eps: float = 1e-5, sum_out=None, out=None):
    """(sum, y): sum = a + b in bf16 (as add), y = rmsnorm(sum, g) (the same
    bits as the two calls).  sum_out may be a or b (in-place residual)."""
    lib = load()
    _check_bf16(a, "a", 2)
    _check_bf16(b, "b", 2)
    _check_bf16(g, "g", 1)
    M, H = a.shape
    if tuple(b.shape) != (M, H) or g.shape[0] != H:
        raise ValueError("a, b must be [M,H] and the gain [H]")
    if sum_out is None:
        sum_out = torch.empty_like(a)
    if out is None:
        out = torch.empty_like(a)
    for t, name in ((sum_out, "sum_out"), (out, "out")):
        _check_bf16(t, name, 2)
        if tuple(t.shape) != (M, H):
            raise ValueError(f"{name} has the wrong shape")
    st = lib.bi_add_rmsnorm(a.data_ptr(), b.data_ptr(), g.data_ptr(), sum_out.data_ptr(),
                            out.data_ptr(), M, H, ctypes.c_float(eps), _stream(a.device))
    _raise(st, "bi_add_rmsnorm")
    return sum_out, out


def _attn_desc(q, kv, block_table, max_ctx_len, scale, table_rows=None):
    B, Hq, D = q.shape
    P, two, Hkv, PS, D2 = kv.shape
    if two != 2 or D2 != D:
        raise ValueError("kv_pages must be [P, 2, Hkv, page_size, head_dim]")
    if block_table.dim() != 2 or block_table.shape[0] != (B if table_rows is None else table_rows):
        raise ValueError("block_table must be [batch, max_blocks]")
    if scale is None:
        scale = 0.0          # the library's default, 1/sqrt(head_dim)
    return AttnDesc(B, Hq, Hkv, D, PS, block_table.shape[1], P, int(max_ctx_len), scale)


def attn_workspace_bytes(desc: AttnDesc) -> int:
    return int(load().bi_attn_workspace_bytes(ctypes.byref(desc)))


def attn_fast_workspace_bytes(desc: AttnDesc) -> int:
    return int(load().bi_attn_fast_workspace_bytes(ctypes.byref(desc)))


def _attn(fn_name, wsq, q, kv, block_table, ctx_lens, max_ctx_len, scale, out, ws):
    lib = load()
    _check_bf16(q, "q", 3)
    _check_bf16(kv, "kv_pages", 5)
    for t, n in ((block_table, "block_table"), (ctx_lens, "ctx_lens")):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 device tensor")
    if ctx_lens.dim() != 1 or ctx_lens.shape[0] != q.shape[0]:
        raise ValueError("ctx_lens must be [batch]")
    if max_ctx_len is None:
        max_ctx_len = int(ctx_lens.max().item())  # host sync; pass it to avoid one
    desc = _attn_desc(q, kv, block_table, max(int(max_ctx_len), 1), scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_bf16(out, "out", 3)
        if out.shape != q.shape:
            raise ValueError("out has the wrong shape")
    need = int(getattr(lib, wsq)(ctypes.byref(desc)))
    buf = _ws_for(q.device, ws).get(need)
    st = getattr(lib, fn_name)(q.data_ptr(), kv.data_ptr(), block_table.data_ptr(),
                               ctx_lens.data_ptr(), out.data_ptr(), ctypes.byref(desc),
                               buf.data_ptr(), buf.numel(), _stream(q.device))
    _raise(st, fn_name)
    return out


def paged_decode_attn(q, kv_pages, block_table, ctx_lens, max_ctx_len=None, scale=None,
                      out=None, ws: Workspace | None = None):
    """Batch-invariant paged decode attention (fixed 256-token chunks)."""
    return _attn("bi_paged_decode_attn", "bi_attn_workspace_bytes", q, kv_pages, block_table,
                 ctx_lens, max_ctx_len, scale, out, ws)


def paged_decode_attn_fast(q, kv_pages, block_table, ctx_lens, max_ctx_len=None, scale=None,
                           out=None, ws: Workspace | None = None):
    """Paged decode attention with batch-dependent splits (not batch-invariant)."""
    return _attn("bi_paged_decode_attn_fast", "bi_attn_fast_workspace_bytes", q, kv_pages,
                 block_table, ctx_lens, max_ctx_len, scale, out, ws)


# ---------------------------------------------------------------------------
# Decoder-layer element-wise steps
# ---------------------------------------------------------------------------

def _check_i32(t: torch.Tensor, name: str):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 device tensor")


def embed(tokens, table, out=None):
    """out[m] = table[tokens[m]] (ids outside the table give zero rows)."""
    lib = load()
    _check_i32(tokens, "tokens")
    _check_bf16(table, "table", 2)
    M, (V, H) = tokens.shape[0], table.shape
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=table.device)
    _raise(lib.bi_embed(tokens.data_ptr(), table.data_ptr(), out.data_ptr(), M, V, H,
                        _stream(table.device)), "bi_embed")
    return out


def rope_table(theta: float, head_dim: int, max_pos: int, device="cuda"):
    """(cos, sin) float32 device tensors [max_pos, head_dim/2] built by the
    library on the host (angle in double, one rounding to fp32 each)."""
    lib = load()
    c = torch.empty((max_pos, head_dim // 2), dtype=torch.float32)
    s = torch.empty_like(c)
    _raise(lib.bi_rope_table(ctypes.c_double(theta), head_dim, max_pos, c.data_ptr(),
                             s.data_ptr()), "bi_rope_table")
    return c.to(device), s.to(device)


def rope(x, heads: int, pos, cos_t, sin_t, out=None):
    """RoPE of the first heads*128 values of each row of x ([M, >= heads*128]
    bf16, rows may be strided, e.g. a slice of a fused q|k|v row)."""
    lib = load()
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise TypeError("x must be a 2-D bf16 device tensor with unit column stride")
    _check_i32(pos, "pos")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, heads, 128), dtype=torch.bfloat16, device=x.device)
    for t, n in ((cos_t, "cos"), (sin_t, "sin")):
        if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{n} table must be a contiguous float32 device tensor")
    _raise(lib.bi_rope(x.data_ptr(), x.stride(0), out.data_ptr(), pos.data_ptr(),
                       cos_t.data_ptr(), sin_t.data_ptr(), M, heads, 128, cos_t.shape[0],
                       _stream(x.device)), "bi_rope")
    return out


def kv_append(k, v, kv_pages, block_table, pos):
    """Write k, v ([M, >= Hkv*128] bf16, rows may be strided) into their
    cache slots (kv_pages [P, 2, Hkv, 16, 128]); block_table is [M, MB]."""
    lib = load()
    _check_bf16(kv_pages, "kv_pages", 5)
    _check_i32(block_table, "block_table")
    _check_i32(pos, "pos")
    for t, n in ((k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 2 or t.stride(1) != 1:
            raise TypeError(f"{n} must be a 2-D bf16 device tensor with unit column stride")
    P, _, Hkv, PS, D = kv_pages.shape
    _raise(lib.bi_kv_append(k.data_ptr(), k.stride(0), v.data_ptr(), v.stride(0),
                            kv_pages.data_ptr(), block_table.data_ptr(), pos.data_ptr(),
                            k.shape[0], Hkv, D, PS, block_table.shape[1], P,
                            _stream(k.device)), "bi_kv_append")


def silu_mul(gu, out=None):
    """bf16(silu(gate) * up) for gu = [gate | up] of shape [M, 2F]."""
    lib = load()
    _check_bf16(gu, "gu", 2)
    M, F2 = gu.shape
    if out is None:
        out = torch.empty((M, F2 // 2), dtype=torch.bfloat16, device=gu.device)
    _raise(lib.bi_silu_mul(gu.data_ptr(), out.data_ptr(), M, F2 // 2, _stream(gu.device)),
           "bi_silu_mul")
    return out


def add(a, b, out=None):
    """bf16(a + b) element-wise (one fp32 addition)."""
    lib = load()
    for t, n in ((a, "a"), (b, "b")):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous bf16 device tensor")
    if a.shape != b.shape:
        raise ValueError("a and b differ in shape")
    if out is None:
        out = torch.empty_like(a)
    _raise(lib.bi_add(a.data_ptr(), b.data_ptr(), out.data_ptr(), a.numel(), _stream(a.device)),
           "bi_add")
    return out


def paged_prefill_attn(q, kv_pages, block_table, row_start, ctx_lens, max_rows_per_request=None,
                       max_ctx_len=None, scale=None, out=None, ws: Workspace | None = None):
    """Multi-query attention for rows grouped by request (block_table has one
    row per request, row_start [R+1] delimits each request's rows); every row
    gets bitwise the decode entry point's result.  max_rows_per_request
    defaults to the largest request (read back from row_start)."""
    lib = load()
    if max_rows_per_request is None:
        max_rows_per_request = int((row_start[1:] - row_start[:-1]).max().item())
    _check_bf16(q, "q", 3)
    _check_bf16(kv_pages, "kv_pages", 5)
    for t, n in ((block_table, "block_table"), (row_start, "row_start"), (ctx_lens, "ctx_lens")):
        _check_i32(t, n)
    if ctx_lens.shape[0] != q.shape[0]:
        raise ValueError("ctx_lens must be [rows]")
    if max_ctx_len is None:
        max_ctx_len = int(ctx_lens.max().item())
    if row_start.shape[0] != block_table.shape[0] + 1:
        raise ValueError("row_start must be [requests + 1]")
    # the descriptor's batch is the number of rows; the block table has one
    # row per request
    desc = _attn_desc(q, kv_pages, block_table, max(int(max_ctx_len), 1), scale,
                      table_rows=row_start.shape[0] - 1)
    if out is None:
        out = torch.empty_like(q)
    need = int(lib.bi_attn_workspace_bytes(ctypes.byref(desc)))
    buf = _ws_for(q.device, ws).get(need)
    st = lib.bi_paged_prefill_attn(q.data_ptr(), kv_pages.data_ptr(), block_table.data_ptr(),
                                   row_start.data_ptr(), ctx_lens.data_ptr(), out.data_ptr(),
                                   ctypes.byref(desc), block_table.shape[0],
                                   int(max_rows_per_request), buf.data_ptr(), buf.numel(),
                                   _stream(q.device))
    _raise(st, "bi_paged_prefill_attn")
    return out


def gemm_segments(x, W, part=None):
    """Segment sums of x @ W: [ceil(K/512), M, N] float32, segment s over K
    rows [512 s, 512 s + 512), each from +0 (the local half of a K-sharded
    GEMM)."""
    lib = load()
    _check_bf16(x, "x", 2)
    _check_bf16(W, "W", 2)
    M, K = x.shape
    K2, N = W.shape
    if K2 != K:
        raise ValueError("x and W disagree on K")
    S = (K + 511) // 512
    if part is None:
        part = torch.empty((S, M, N), dtype=torch.float32, device=x.device)
    if tuple(part.shape) != (S, M, N) or part.dtype != torch.float32 or not part.is_contiguous():
        raise ValueError("part must be contiguous float32 [ceil(K/512), M, N]")
    st = lib.bi_gemm_segments(x.data_ptr(), W.data_ptr(), part.data_ptr(), M, N, K,
                              _stream(x.device))
    _raise(st, "bi_gemm_segments")
    return part


def gemm_fold(part, y=None):
    """bf16 of the left-to-right fp32 sum of part's segments ([S, M, N])."""
    lib = load()
    if part.dtype != torch.float32 or part.dim() != 3 or not part.is_contiguous():
        raise ValueError("part must be contiguous float32 [S, M, N]")
    S, M, N = part.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=part.device)
    _check_bf16(y, "y", 2)
    st = lib.bi_gemm_fold(part.data_ptr(), y.data_ptr(), M, N, S, _stream(part.device))
    _raise(st, "bi_gemm_fold")
    return y


def sample(logits, seeds, steps, temperature, tokens=None, ws: Workspace | None = None):
    """Per-row token of logits [M, V] (bf16): Gumbel-max with Philox noise
    keyed by (seeds[m], steps[m]) at temperature[m] > 0, else argmax."""
    lib = load()
    _check_bf16(logits, "logits", 2)
    M, V = logits.shape
    for t, n, dt in ((seeds, "seeds", torch.uint64), (steps, "steps", torch.uint64),
                     (temperature, "temperature", torch.float32)):
        if t.dtype != dt or t.shape != (M,) or not t.is_contiguous() or t.device != logits.device:
            raise ValueError(f"{n} must be a contiguous {dt} [M] tensor on the logits' device")
    if tokens is None:
        tokens = torch.empty(M, dtype=torch.int32, device=logits.device)
    need = int(lib.bi_sample_workspace_bytes(M))
    buf = _ws_for(logits.device, ws).get(need)
    st = lib.bi_sample(logits.data_ptr(), M, V, seeds.data_ptr(), steps.data_ptr(),
                       temperature.data_ptr(), tokens.data_ptr(), buf.data_ptr(), buf.numel(),
                       _stream(logits.device))
    _raise(st, "bi_sample")
    return tokens


def verify_commit(candidates, verified, row_start, commit_len):
    """Commit-or-rollback of grouped verification windows; commit_len [R]
    is updated in place.  Returns (accepted [R], fix_token [R])."""
    lib = load()
    for t, n in ((candidates, "candidates"), (verified, "verified"), (row_start, "row_start"),
                 (commit_len, "commit_len")):
        _check_i32(t, n)
    R = row_start.shape[0] - 1
    if commit_len.shape[0] != R or verified.shape != candidates.shape:
        raise ValueError("commit_len must be [R] and verified match candidates")
    acc = torch.empty(R, dtype=torch.int32, device=row_start.device)
    fix = torch.empty(R, dtype=torch.int32, device=row_start.device)
    st = lib.bi_verify_commit(candidates.data_ptr(), verified.data_ptr(), candidates.shape[0],
                              row_start.data_ptr(), R, acc.data_ptr(), commit_len.data_ptr(),
                              fix.data_ptr(), _stream(row_start.device))
    _raise(st, "bi_verify_commit")
    return acc, fix
