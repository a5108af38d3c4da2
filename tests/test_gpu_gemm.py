"""bi_gemm on the GPU: parity with the oracle, bitwise invariance across M,
run-to-run and row order, the ordering pins, and the fast twin."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from invariant_bi_gemm_02_amd import synth
from tolerance import bits_to_f64, check_close_bf16

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


def bits(t):
    return synth.to_bits(t)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def bf16_exact(values):
    f = np.asarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    assert not np.any(u & 0xFFFF)
    return (u >> 16).astype(np.uint16)


def test_config1_rows_at_m1_equal_rows_at_m8(gpu):
    """The Determinism article's section-1 experiment, x[8,4096] . W[4096,4096]
    with N(0,1) bf16 data: the page reports >30% of elements differ between
    batch 1 and batch 8 with cuBLAS; here the share must be exactly 0."""
    with open(os.path.join(GOLDEN, "config1_mismatch.json")) as fh:
        target = json.load(fh)["target_here"]["exact_mismatch_share"]
    x, w = synth.gemm_inputs(8, 4096, 4096, seed=0, w_std=1.0)
    xd, wd = x.to(DEV), w.to(DEV)
    y8 = gpu.gemm(xd, wd)
    y1 = torch.cat([gpu.gemm(xd[i:i + 1].contiguous(), wd) for i in range(8)])
    torch.cuda.synchronize()
    mismatch = (y8.view(torch.int16) != y1.view(torch.int16)).float().mean().item()
    assert mismatch == target
    stats = check_close_bf16(bits(y8), oracle.gemm(bits(x), bits(w)), what="config1")
    print("config1 vs oracle:", stats)


@pytest.mark.parametrize("M,N,K", [
    (1, 64, 32), (1, 192, 544), (5, 128, 1056), (16, 320, 512), (16, 64, 32), (13, 128, 1536),
    (16, 64, 2080), (17, 64, 96),
    (64, 192, 1024), (65, 256, 544), (130, 192, 1056), (300, 320, 96),
    (48, 320, 1056), (33, 128, 608), (40, 64, 96)])
def test_parity_with_oracle_small_shapes(gpu, M, N, K):
    x, w = synth.gemm_inputs(M, K, N, seed=M + N + K, w_std=0.5)
    y = gpu.gemm(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    stats = check_close_bf16(bits(y), oracle.gemm(bits(x), bits(w)), what=f"{M}x{N}x{K}")
    assert stats["bit_equal_share"] > 0.9


@pytest.mark.parametrize("M", [1, 16, 200])
def test_small_integer_inputs_are_bit_exact(gpu, M):
    """Integers in [-3, 3] keep every partial sum exact, so any association
    gives the same value: GPU = oracle = fp64, bitwise."""
    K, N = 1056, 192
    rng = np.random.default_rng(M)
    xf = rng.integers(-3, 4, size=(M, K)).astype(np.float32)
    wf = rng.integers(-3, 4, size=(K, N)).astype(np.float32)
    x, w = bf16_exact(xf), bf16_exact(wf)
    y = gpu.gemm(synth.from_bits(x, DEV), synth.from_bits(w, DEV))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(y), oracle.gemm(x, w))
    np.testing.assert_array_equal(bits_to_f64(bits(y)),
                                  bits_to_f64(oracle.gemm(x, w)))


BIG = 2.0 ** 13


def ordering_case(K, placements, M, row):
    x = np.zeros((M, K), np.float32)
    x[:] = 0.0
    w = np.zeros((K, 64), np.float32)
    for k, (xv, wv) in placements.items():
        x[row, k] = xv
        w[k, 0] = wv
    return bf16_exact(x), bf16_exact(w)


@pytest.mark.parametrize("M,row", [(1, 0), (40, 37), (130, 129)])
@pytest.mark.parametrize("ks,expect", [
    ((0, 512, 1024), 1.0),    # one product per segment, folded 0, 1, 2
    ((1024, 512, 0), 0.0),    # reversed: the fold is fp32 round-to-nearest
    ((0, 32, 64), 1.0),       # one product per K-block of one segment
])
def test_ordering_pins(gpu, M, row, ks, expect):
    """The page's 1e8 example made bf16-exact: products 2^26, -2^26, 1.  The
    fixed order gives exactly 1.0 on both paths (split and tile)."""
    vals = [(BIG, BIG), (-BIG, BIG), (1.0, 1.0)]
    x, w = ordering_case(1536, dict(zip(ks, vals)), M, row)
    y = gpu.gemm(synth.from_bits(x, DEV), synth.from_bits(w, DEV))
    torch.cuda.synchronize()
    yf = bits_to_f64(bits(y))
    assert yf[row, 0] == expect
    assert np.all(yf[:, 1:] == 0)


@pytest.mark.parametrize("M,row", [(1, 0), (130, 5)])
def test_segment_starts_from_zero(gpu, M, row):
    """Segment 1 holds -2^26 then +1 (two K-blocks).  Started from +0 the
    segment sum loses the 1, so the fold cannot give 1.0; carrying the
    running sum into segment 1 would give exactly 1.0."""
    x, w = ordering_case(1024, {0: (BIG, BIG), 512: (-BIG, BIG), 544: (1.0, 1.0)}, M, row)
    y = gpu.gemm(synth.from_bits(x, DEV), synth.from_bits(w, DEV))
    torch.cuda.synchronize()
    v = bits_to_f64(bits(y))[row, 0]
    assert v != 1.0
    assert abs(v) <= 8.0


def test_inblock_probe_is_recorded(gpu):
    """Three products in one 32-deep block: the oracle's left-to-right model
    gives 0.0; the matrix core's own grouping is recorded, not asserted."""
    x, w = ordering_case(32, {0: (1.0, 1.0), 1: (BIG, BIG), 2: (-BIG, BIG)}, 1, 0)
    y = gpu.gemm(synth.from_bits(x, DEV), synth.from_bits(w, DEV))
    torch.cuda.synchronize()
    print("in-block (1, 2^26, -2^26) on the matrix core ->", bits_to_f64(bits(y))[0, 0])


@pytest.mark.parametrize("name,K,N", synth.LLAMA3_8B_LINEARS)
def test_m_sweep_bitwise_and_sampled_oracle(gpu, name, K, N):
    """Every M in the sweep reproduces the leading rows of the M=2048 run bit
    for bit; sampled rows of the full-size runs agree with the oracle."""
    x, w = synth.gemm_inputs(2048, K, N, seed=3, device=DEV)
    ref = gpu.gemm(x, w)
    for M in synth.M_SWEEP:
        y = gpu.gemm(x[:M].contiguous(), w)
        assert same_bits(y, ref[:M]), f"{name}: M={M} differs from the M=2048 rows"
    torch.cuda.synchronize()
    rows = [0, 1, 1000, 2047]
    got = bits(ref[rows])
    want = oracle.gemm(bits(x[rows]), bits(w))
    check_close_bf16(got, want, what=f"{name} sampled rows")


@pytest.mark.parametrize("name,K,N", synth.LLAMA3_8B_LINEARS)
def test_every_m_from_1_to_2048_bitwise(gpu, name, K, N):
    """Every M from 1 to 2048, not only the sweep's: the leading M rows of
    the M = 2048 run, bit for bit.  This crosses every boundary of the plan
    on each linear (skinny kernel at 16/32/64 rows, 128 x 128 tiles for wide N
    at 16-64 rows, K-slice, 64 x 128 and 128 x 128 register-fold tiles,
    256 x 128 tiles with and without a re-tiled last round, 256 x 192 whole
    rounds).  Mismatch flags stay on the device until the end."""
    x, w = synth.gemm_inputs(2048, K, N, seed=13, device=DEV)
    ref = gpu.gemm(x, w)
    ref16 = ref.view(torch.int16)
    flags = []
    for M in range(1, 2049):
        y = gpu.gemm(x[:M].contiguous(), w)
        flags.append((y.view(torch.int16) != ref16[:M]).any())
    bad = torch.stack(flags).nonzero().flatten().add(1).tolist()
    assert not bad, f"{name}: M = {bad[:10]} differ from the M = 2048 rows"


@pytest.mark.parametrize("M,N,K", [(2048, 3136, 544), (1500, 4224, 1056), (700, 8256, 96),
                                   (2048, 3136, 640), (2048, 3136, 576), (1500, 4224, 1216)])
def test_tile_path_ragged_shapes(gpu, M, N, K):
    """Tile-path launches whose last tile column is half empty (N % 128 == 64),
    whose tile count is not a multiple of the 8 XCDs, and whose K ends in a
    half stage (K % 64 == 32), in one whole stage (K % 512 == 64) or in a
    partial segment of two or three stages (K % 512 == 128, 192): sampled rows
    match the skinny path bit for bit and the oracle within tolerance."""
    x, w = synth.gemm_inputs(M, K, N, seed=M + K, device=DEV)
    y = gpu.gemm(x, w)
    rows = [0, 1, M // 2, M - 1]
    for r in rows:
        assert same_bits(gpu.gemm(x[r:r + 1].contiguous(), w), y[r:r + 1]), f"row {r}"
    torch.cuda.synchronize()
    check_close_bf16(bits(y[rows]), oracle.gemm(bits(x[rows]), bits(w)), what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(200, 4160, 14432), (256, 4096, 14656), (300, 4032, 14336)])
def test_slice_path_runs_of_segments(gpu, M, N, K):
    """Mid-size M with few tiles: one workgroup runs several consecutive
    512-row segments and stores each segment's sum.  The shapes give 2, 4 and
    7 segments per workgroup with a last run of one segment (29 segments), a
    last segment of 1.5 and 5 stages, a half-empty last tile column and a
    second tile row of 44 rows.  The workspace is filled with NaN first, so a
    sum that is not stored cannot pass on stale values.  Every row of the
    first 64 matches the skinny path bit for bit (one call at M = 64), sampled
    rows match single-row calls, and the oracle within tolerance."""
    x, w = synth.gemm_inputs(M, K, N, seed=M + N + K, device=DEV)
    ws = gpu.Workspace(DEV)
    ws.get(gpu.gemm_workspace_bytes(M, N, K)).view(torch.float32).fill_(float("nan"))
    y = gpu.gemm(x, w, ws=ws)
    assert same_bits(gpu.gemm(x[:64].contiguous(), w), y[:64])
    rows = [0, 100, M - 1]
    for r in rows:
        assert same_bits(gpu.gemm(x[r:r + 1].contiguous(), w), y[r:r + 1]), f"row {r}"
    torch.cuda.synchronize()
    assert not torch.isnan(y.float()).any()
    check_close_bf16(bits(y[rows]), oracle.gemm(bits(x[rows]), bits(w)), what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1000, 4096, 14336), (1025, 4032, 4640), (520, 6144, 1056),
                                   (777, 4160, 4096)])
def test_fold128_path_ragged_shapes(gpu, M, N, K):
    """The 128 x 128 register-fold path (256 x 128 tiles too few, 128 x 128
    tiles enough to fill the chip): a last tile row of 104, 1, 8 and 9 rows,
    a last tile column of 64 columns (N % 128 == 64), K ending in a short
    segment of one K-block (K % 512 == 32).  Every row of the first 64 matches the
    skinny path bit for bit (one call at M = 64), sampled rows match
    single-row calls, and the oracle within tolerance."""
    x, w = synth.gemm_inputs(M, K, N, seed=M * 3 + K, device=DEV)
    assert gpu.gemm_workspace_bytes(M, N, K) == 0      # every segment stays in registers
    y = gpu.gemm(x, w)
    assert same_bits(gpu.gemm(x[:64].contiguous(), w), y[:64])
    rows = [0, 127, 128, M // 2, M - 1]
    for r in rows:
        assert same_bits(gpu.gemm(x[r:r + 1].contiguous(), w), y[r:r + 1]), f"row {r}"
    torch.cuda.synchronize()
    check_close_bf16(bits(y[rows]), oracle.gemm(bits(x[rows]), bits(w)), what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(512, 4096, 14336), (330, 4160, 4640), (257, 6144, 1056),
                                   (640, 4032, 4096)])
def test_fold64_path_ragged_shapes(gpu, M, N, K):
    """The 64 x 128 register-fold path (tiles of 256 and of 128 rows too few
    to fill the chip, tiles of 64 rows enough): down at M = 512, then a last
    tile row of 10, 1 and 64 rows, a last tile column of 64 columns
    (N % 128 == 64) and a one-K-block last segment (K % 512 == 32).  Every
    row of the first 64 matches the skinny path bit for bit (one call at
    M = 64), sampled rows match single-row calls, and the oracle within
    tolerance."""
    x, w = synth.gemm_inputs(M, K, N, seed=M * 5 + K, device=DEV)
    assert gpu.gemm_workspace_bytes(M, N, K) == 0      # every segment stays in registers
    y = gpu.gemm(x, w)
    assert same_bits(gpu.gemm(x[:64].contiguous(), w), y[:64])
    rows = [0, 63, 64, M // 2, M - 1]
    for r in rows:
        assert same_bits(gpu.gemm(x[r:r + 1].contiguous(), w), y[r:r + 1]), f"row {r}"
    torch.cuda.synchronize()
    check_close_bf16(bits(y[rows]), oracle.gemm(bits(x[rows]), bits(w)), what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(2048, 6144, 4096), (2000, 6144, 4128), (1024, 28672, 4096),
                                   (1536, 6144, 4096), (1100, 7104, 1056)])
def test_partial_round_retiled(gpu, M, N, K):
    """256 x 128 tiles that leave a partial last round on 256 CUs.  At
    N = 6144 and 8 tile rows, 256 x 192 tiles make one whole round and run
    instead (the second shape with a last tile row of 208 rows and a
    one-K-block last segment).  Otherwise (896, 288 and 280 tiles) the tile
    columns of the last round run as 128 x 128 tiles in a second launch; the
    last shape has a last tile row of 76 rows, a last tile column of 64
    columns and a one-K-block last segment.  Rows match the skinny path and
    single-row calls bit for bit, across the seam between the two launches'
    columns where there is one, and the oracle within tolerance."""
    x, w = synth.gemm_inputs(M, K, N, seed=M + 7 * K, device=DEV)
    assert gpu.gemm_workspace_bytes(M, N, K) == 0
    y = gpu.gemm(x, w)
    assert same_bits(gpu.gemm(x[:64].contiguous(), w), y[:64])
    rows = [0, 255, 256, M // 2, M - 1]
    for r in rows:
        assert same_bits(gpu.gemm(x[r:r + 1].contiguous(), w), y[r:r + 1]), f"row {r}"
    torch.cuda.synchronize()
    check_close_bf16(bits(y[rows]), oracle.gemm(bits(x[rows]), bits(w)), what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_vs_oracle_and_single_rows(gpu, seed):
    """Seeded random shapes (M 1-299, N a multiple of 64 up to 1024, K a
    multiple of 32 up to 2048, so every path below M = 300 and ragged last
    segments come up): within tolerance of the oracle, and sampled rows
    computed alone bitwise equal to their rows in the batch."""
    rng = np.random.default_rng(300 + seed)
    M = int(rng.integers(1, 300))
    N = 64 * int(rng.integers(1, 17))
    K = 32 * int(rng.integers(1, 65))
    x, w = synth.gemm_inputs(M, K, N, seed=700 + seed, w_std=0.5)
    xd, wd = x.to(DEV), w.to(DEV)
    y = gpu.gemm(xd, wd)
    torch.cuda.synchronize()
    check_close_bf16(bits(y), oracle.gemm(bits(x), bits(w)), what=f"{M}x{N}x{K}")
    for r in sorted({0, M - 1, int(rng.integers(0, M))}):
        assert same_bits(gpu.gemm(xd[r:r + 1].contiguous(), wd), y[r:r + 1]), f"row {r}"


@pytest.mark.parametrize("M,N,K", [(16, 28672, 4096), (17, 24640, 1056), (40, 25600, 4640),
                                   (64, 28672, 14336), (48, 49216, 4096)])
def test_decode_rows_on_fold128_tiles(gpu, M, N, K):
    """16-64 rows with wide N (at least 192 tiles of 128 x 128: gate_up, an
    vocabulary-wide LM head) run on the 128 x 128 register-fold tiles instead of the skinny
    kernel; shapes with a half-empty last tile column (N % 128 == 64) and a
    one-K-block last segment included.  Every row matches the same row
    computed alone (the skinny path) bit for bit, and sampled rows the
    oracle within tolerance."""
    x, w = synth.gemm_inputs(M, K, N, seed=M * 7 + K, device=DEV)
    assert gpu.gemm_workspace_bytes(M, N, K) == 0
    y = gpu.gemm(x, w)
    for r in range(M):
        assert same_bits(gpu.gemm(x[r:r + 1].contiguous(), w), y[r:r + 1]), f"row {r}"
    torch.cuda.synchronize()
    rows = [0, M // 2, M - 1]
    check_close_bf16(bits(y[rows]), oracle.gemm(bits(x[rows]), bits(w)), what=f"{M}x{N}x{K}")


def test_run_to_run_and_row_permutation(gpu):
    x, w = synth.gemm_inputs(300, 4096, 4096, seed=4, device=DEV)
    base = gpu.gemm(x, w)
    for _ in range(10):
        assert same_bits(gpu.gemm(x, w), base)
    perm = torch.randperm(300, generator=torch.Generator().manual_seed(0)).to(DEV)
    yp = gpu.gemm(x[perm].contiguous(), w)
    assert same_bits(yp, base[perm])
    small = gpu.gemm(x[:7].contiguous(), w)
    for _ in range(10):
        assert same_bits(gpu.gemm(x[:7].contiguous(), w), small)


@pytest.mark.parametrize("M,N", [(1, 4096), (16, 4096), (64, 4096), (300, 4096), (2048, 4096),
                                 (2048, 6208), (600, 28672), (1025, 6144)])
def test_fast_twin_parity(gpu, M, N):
    """The fast twin on each of its paths (skinny; K-slice at M = 300;
    256 x 128 tiles; 256 x 256 tiles, with a last tile column of 64 columns
    at N = 6208 and a last tile row of 88 rows at M = 600), within tolerance
    of the oracle."""
    K = 4096
    x, w = synth.gemm_inputs(M, K, N, seed=5, device=DEV)
    y = gpu.gemm_fast(x, w)
    torch.cuda.synchronize()
    rows = sorted(set([0, M // 2, M - 1]))
    check_close_bf16(bits(y[rows]), oracle.gemm(bits(x[rows]), bits(w)), what=f"fast M={M}")


def test_special_values_are_row_invariant(gpu):
    """x rows holding +-inf, NaN, -0 and subnormal bf16 values: every row at
    M = 1 (skinny path), inside M = 200 (slice path) and inside M = 2048
    (tile path) gives the same bits, including NaN and infinity results."""
    K, N = 4096, 4096
    x = synth.bf16_normal((2048, K), seed=21, device=DEV)
    w = synth.bf16_normal((K, N), seed=22, std=0.02, device=DEV)
    xb = x.view(torch.int16)
    special = torch.tensor([0x7F80, -128, 0x7FC0, -32768, 0x0001, -32767], dtype=torch.int16,
                           device=DEV)                       # +inf -inf nan -0 sub -sub
    for i, v in enumerate(special):
        xb[3 * i + 1, 100 * i + 7] = v
        xb[3 * i + 2, :] = v if i in (3, 4, 5) else xb[3 * i + 2, :]
    full = gpu.gemm(x, w)
    mid = gpu.gemm(x[:200].contiguous(), w)
    torch.cuda.synchronize()
    assert same_bits(mid, full[:200])
    for r in range(20):
        one = gpu.gemm(x[r:r + 1].contiguous(), w)
        torch.cuda.synchronize()
        assert same_bits(one, full[r:r + 1]), r
    # the rows with an infinity or NaN produce non-finite outputs
    f = full.float()
    assert torch.isinf(f[1]).any() or torch.isnan(f[1]).any()
    assert torch.isnan(f[7]).any()
