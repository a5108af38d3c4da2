"""The C-ABI library loads, exports every symbol include/bi.h declares, and
rejects bad arguments before touching the GPU (these calls never reach a
launch, so they run without one)."""
import ctypes
import os
import re

import pytest

import invariant_bi_gemm_02_amd as bi
from invariant_bi_gemm_02_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bi.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libbi.so is not built (run __graft_entry__.build())")
    return bi.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), f"{n} declared in bi.h but not exported"
    assert set(names) == set(_lib.EXPORTS)


def test_version_names_target_and_schedule(lib):
    v = bi.version()
    assert "gfx950" in v and "KC=512" in v and "chunk=256" in v


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert lib.bi_status_string(code)
    assert lib.bi_status_string(-6) != lib.bi_status_string(-99)


def test_noalloc_argument_checks(lib):
    """bi_gemm_noalloc runs bi_gemm's checks, then refuses a call whose
    workspace would exceed the static scratch, all before touching a device."""
    ok = 0x1000
    assert lib.bi_gemm_noalloc(None, P(ok), P(ok), 1, 64, 32, None) == -1
    assert lib.bi_gemm_noalloc(P(ok), P(ok), P(ok), 0, 64, 32, None) == -2
    assert lib.bi_gemm_noalloc(P(ok), P(ok), P(ok), 1, 64, 33, None) == -3
    assert lib.bi_gemm_noalloc(P(ok + 2), P(ok), P(ok), 1, 64, 32, None) == -3
    assert lib.bi_gemm_workspace_bytes(64, 16384, 14336) > (64 << 20)
    assert lib.bi_gemm_noalloc(P(ok), P(ok), P(ok), 64, 16384, 14336, None) == -6


def P(v):
    return ctypes.c_void_p(v)


def test_ceiling_read_argument_checks(lib):
    """The streaming-read helper refuses bad arguments before touching a
    device."""
    ok = 0x1000
    assert lib.bi_ceiling_read(None, 16, P(ok), None) == -1
    assert lib.bi_ceiling_read(P(ok), 16, None, None) == -1
    assert lib.bi_ceiling_read(P(ok), 0, P(ok), None) == -2
    assert lib.bi_ceiling_read(P(ok), (1 << 40) + 16, P(ok), None) == -2
    assert lib.bi_ceiling_read(P(ok), 24, P(ok), None) == -3
    assert lib.bi_ceiling_read(P(ok + 8), 16, P(ok), None) == -3
    assert lib.bi_ceiling_read(P(ok), 16, P(ok + 2), None) == -3


def test_gemm_argument_checks(lib):
    ok = 0x1000
    assert lib.bi_gemm(None, P(ok), P(ok), 1, 64, 32, None, 0, None) == -1
    assert lib.bi_gemm(P(ok), P(ok), P(ok), 0, 64, 32, None, 0, None) == -2
    assert lib.bi_gemm(P(ok), P(ok), P(ok), 1, 64, 33, None, 0, None) == -3   # K % 32
    assert lib.bi_gemm(P(ok), P(ok), P(ok), 1, 48, 32, None, 0, None) == -3   # N % 64
    assert lib.bi_gemm(P(ok + 2), P(ok), P(ok), 1, 64, 32, None, 0, None) == -3  # alignment
    assert lib.bi_gemm(P(ok), P(ok), P(ok), 1 << 20, 1 << 12, 1 << 12, None, 0, None) == -2
    # M <= 64 sends segment sums through the workspace
    need = lib.bi_gemm_workspace_bytes(32, 4096, 4096)
    assert need == 8 * 32 * 4096 * 4
    assert lib.bi_gemm(P(ok), P(ok), P(ok), 32, 4096, 4096, P(ok), need - 16, None) == -4
    assert lib.bi_gemm(P(ok), P(ok), P(ok), 32, 4096, 4096, None, 0, None) == -4
    # decode-sized M: segment sums go through the workspace, except at 16-64
    # rows with enough 128 x 128 tiles to fill the chip; mid M with too few
    # tiles of 128 and of 64 rows slices K through the workspace; larger M
    # folds in registers
    assert lib.bi_gemm_workspace_bytes(1, 4096, 4096) == 8 * 1 * 4096 * 4
    assert lib.bi_gemm_workspace_bytes(16, 4096, 14336) == 28 * 16 * 4096 * 4
    assert lib.bi_gemm_workspace_bytes(15, 28672, 4096) == 8 * 15 * 28672 * 4
    assert lib.bi_gemm_workspace_bytes(16, 28672, 4096) == 0
    assert lib.bi_gemm_workspace_bytes(64, 16384, 4096) == 8 * 64 * 16384 * 4
    assert lib.bi_gemm_workspace_bytes(64, 24576, 4096) == 0
    assert lib.bi_gemm_workspace_bytes(256, 4096, 14336) == 28 * 256 * 4096 * 4
    assert lib.bi_gemm_workspace_bytes(512, 4096, 14336) == 0      # 256 tiles of 64 x 128
    assert lib.bi_gemm_workspace_bytes(1024, 4096, 14336) == 0     # 256 tiles of 128 x 128
    assert lib.bi_gemm_workspace_bytes(2048, 4096, 4096) == 0


def test_segment_and_fold_argument_checks(lib):
    ok = 0x1000
    assert lib.bi_gemm_segments(None, P(ok), P(ok), 1, 64, 512, None) == -1
    assert lib.bi_gemm_segments(P(ok), P(ok), P(ok), 1, 64, 33, None) == -3   # K % 32
    assert lib.bi_gemm_segments(P(ok), P(ok), P(ok), 0, 64, 512, None) == -2
    assert lib.bi_gemm_fold(None, P(ok), 1, 64, 1, None) == -1
    assert lib.bi_gemm_fold(P(ok), P(ok), 1, 64, 0, None) == -2
    assert lib.bi_gemm_fold(P(ok), P(ok), 70000, 64, 1, None) == -2           # M > 65535
    assert lib.bi_gemm_fold(P(ok), P(ok), 1, 96, 1, None) == -3               # N % 64
    assert lib.bi_gemm_fold(P(ok + 4), P(ok), 1, 64, 1, None) == -3           # alignment


def test_sample_and_commit_argument_checks(lib):
    ok = 0x1000
    need = lib.bi_sample_workspace_bytes(3)
    assert need == 3 * 32 * 8
    assert lib.bi_sample(None, 1, 10, P(ok), P(ok), P(ok), P(ok), P(ok), need, None) == -1
    assert lib.bi_sample(P(ok), 0, 10, P(ok), P(ok), P(ok), P(ok), P(ok), need, None) == -2
    assert lib.bi_sample(P(ok), 1, 10, P(ok + 4), P(ok), P(ok), P(ok), P(ok), need,
                         None) == -3                                    # seeds % 8
    assert lib.bi_sample(P(ok), 3, 10, P(ok), P(ok), P(ok), P(ok), P(ok), need - 8, None) == -4
    assert lib.bi_verify_commit(P(ok), None, 4, P(ok), 1, P(ok), P(ok), P(ok), None) == -1
    assert lib.bi_verify_commit(P(ok), P(ok), 4, P(ok), 0, P(ok), P(ok), P(ok), None) == -2
    assert lib.bi_verify_commit(P(ok), P(ok), 4, P(ok + 2), 1, P(ok), P(ok), P(ok), None) == -3


def test_workspace_size_counts_segments(lib):
    a = lib.bi_gemm_workspace_bytes(40, 4096, 4096)
    b = lib.bi_gemm_workspace_bytes(40, 4096, 14336)
    assert a == 8 * 40 * 4096 * 4
    assert b == 28 * 40 * 4096 * 4


def test_rmsnorm_argument_checks(lib):
    ok = 0x1000
    f = ctypes.c_float(1e-5)
    assert lib.bi_rmsnorm(None, P(ok), P(ok), 1, 4096, f, None) == -1
    assert lib.bi_rmsnorm(P(ok), P(ok), P(ok), 1, 0, f, None) == -2
    assert lib.bi_rmsnorm(P(ok), P(ok), P(ok), 1, 4100, f, None) == -3
    assert lib.bi_rmsnorm_fast(P(ok), P(ok), P(ok), -1, 4096, f, None) == -2


def test_attention_argument_checks(lib):
    ok = 0x1000
    d = _lib.AttnDesc(4, 32, 8, 128, 16, 64, 1000, 1024, 0.088)
    args = [P(ok), P(ok), P(ok), P(ok), P(ok)]
    need = lib.bi_attn_workspace_bytes(ctypes.byref(d))
    assert need == 4 * 32 * 4 * 132 * 4
    assert lib.bi_paged_decode_attn(*args, ctypes.byref(d), P(ok), need - 4, None) == -4
    bad = _lib.AttnDesc(4, 32, 8, 64, 16, 64, 1000, 1024, 0.088)       # head_dim 64
    assert lib.bi_paged_decode_attn(*args, ctypes.byref(bad), P(ok), 1 << 30, None) == -3
    bad = _lib.AttnDesc(4, 32, 8, 128, 16, 8, 1000, 1024, 0.088)       # table too narrow
    assert lib.bi_paged_decode_attn(*args, ctypes.byref(bad), P(ok), 1 << 30, None) == -2
    bad = _lib.AttnDesc(4, 24, 8, 128, 16, 64, 1000, 1024, 0.088)      # group of 3
    assert lib.bi_paged_decode_attn(*args, ctypes.byref(bad), P(ok), 1 << 30, None) == -3
    assert lib.bi_paged_decode_attn(None, *args[1:], ctypes.byref(d), P(ok), need, None) == -1
    # multi-query entry: [rows] q with a [requests] block table and row_start
    pre = [P(ok), P(ok), P(ok), P(ok), P(ok), P(ok)]
    assert lib.bi_paged_prefill_attn(*pre, ctypes.byref(d), 2, 4, P(ok), need - 4, None) == -4
    assert lib.bi_paged_prefill_attn(*pre[:3], None, *pre[4:], ctypes.byref(d), 2, 4, P(ok),
                                     need, None) == -1
    assert lib.bi_paged_prefill_attn(*pre, ctypes.byref(d), 0, 4, P(ok), need, None) == -2
    assert lib.bi_paged_prefill_attn(*pre, ctypes.byref(d), 2, 5, P(ok), need, None) == -2
    assert lib.bi_paged_prefill_attn(*pre, ctypes.byref(bad), 2, 4, P(ok), need, None) == -3


def test_static_lint_no_float_atomics_or_cu_count_in_invariant_paths():
    """Code-review rule of the Determinism article (section 8): no float
    atomics, and no reduction order that depends on the number of compute
    units.  Float atomics are banned everywhere; the CU count may be read
    only by the fast twins' planners."""
    csrc = os.path.join(ROOT, "invariant_bi_gemm_02_amd", "csrc")
    for fn in os.listdir(csrc):
        text = open(os.path.join(csrc, fn)).read()
        assert not re.search(r"atomicAdd\s*\(\s*\(?\s*float", text), fn
        assert "unsafeAtomicAdd" not in text, fn
        assert "__hip_atomic" not in text and "atomicAdd" not in text, fn
        if "MultiprocessorCount" in text or "multiProcessorCount" in text:
            assert fn == "bi_api.hip", fn


def test_layer_step_argument_checks(lib):
    ok = 1 << 20  # a 16-byte aligned non-null address; never dereferenced on error paths
    P = ctypes.c_void_p
    f = ctypes.c_float(1e-5)
    assert lib.bi_add_rmsnorm(P(ok), None, P(ok), P(ok), P(ok), 1, 4096, f, None) == -1
    assert lib.bi_add_rmsnorm(P(ok), P(ok), P(ok), None, P(ok), 1, 4096, f, None) == -1
    assert lib.bi_add_rmsnorm(P(ok), P(ok), P(ok), P(ok), P(ok), 0, 4096, f, None) == -2
    assert lib.bi_add_rmsnorm(P(ok), P(ok), P(ok), P(ok), P(ok), 1, 4100, f, None) == -3  # H % 8
    assert lib.bi_add_rmsnorm(P(ok), P(ok), P(ok), P(ok), P(ok), 1, 8200, f, None) == -3  # H > 8192
    assert lib.bi_add_rmsnorm(P(ok), P(ok + 2), P(ok), P(ok), P(ok), 1, 4096, f, None) == -3
    assert lib.bi_embed(None, P(ok), P(ok), 1, 10, 64, None) == -1
    assert lib.bi_embed(P(ok), P(ok), P(ok), 0, 10, 64, None) == -2
    assert lib.bi_embed(P(ok), P(ok), P(ok), 1, 10, 60, None) == -3      # H % 8
    assert lib.bi_rope(P(ok), 512, P(ok), P(ok), P(ok), P(ok), 1, 4, 64, 8, None) == -3  # D
    assert lib.bi_rope(P(ok), 256, P(ok), P(ok), P(ok), P(ok), 1, 4, 128, 8, None) == -2  # stride
    assert lib.bi_rope(P(ok), 512, None, P(ok), P(ok), P(ok), 1, 4, 128, 8, None) == -1
    assert lib.bi_rope(P(ok), 514, P(ok), P(ok), P(ok), P(ok), 1, 4, 128, 8, None) == -3  # stride % 4
    assert lib.bi_rope(P(ok + 4), 512, P(ok), P(ok), P(ok), P(ok), 1, 4, 128, 8, None) == -3
    assert lib.bi_kv_append(P(ok), 1024, P(ok), 1024, P(ok), P(ok), P(ok), 1, 8, 128, 32, 4, 4,
                            None) == -3                                  # page size
    assert lib.bi_kv_append(P(ok), 1028, P(ok), 1024, P(ok), P(ok), P(ok), 1, 8, 128, 16, 4, 4,
                            None) == -3                                  # stride % 8
    assert lib.bi_kv_append(P(ok), 512, P(ok), 1024, P(ok), P(ok), P(ok), 1, 8, 128, 16, 4, 4,
                            None) == -2                                  # stride < Hkv*D
    assert lib.bi_silu_mul(P(ok), P(ok), 1, 12, None) == -3
    assert lib.bi_silu_mul(P(ok), P(ok), 0, 16, None) == -2
    assert lib.bi_add(P(ok), P(ok + 2), P(ok), 16, None) == -3
    assert lib.bi_add(P(ok), P(ok), P(ok), 0, None) == -2


def test_rope_table_matches_its_definition(lib):
    """The host-side table: position 0 is (1, 0); column 0 turns one radian
    per position (cos 1 and sin 1 to fp32)."""
    import numpy as np
    c = np.empty((4, 64), np.float32)
    s = np.empty_like(c)
    assert lib.bi_rope_table(5e5, 128, 4, c.ctypes.data, s.ctypes.data) == 0
    assert np.all(c[0] == 1) and np.all(s[0] == 0)
    assert c[1, 0] == np.float32(0.5403023058681398) and s[1, 0] == np.float32(0.8414709848078965)
    assert lib.bi_rope_table(-1.0, 128, 4, c.ctypes.data, s.ctypes.data) == -2
    assert lib.bi_rope_table(5e5, 127, 4, c.ctypes.data, s.ctypes.data) == -2
