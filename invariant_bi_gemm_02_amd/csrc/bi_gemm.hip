// bi_gemm.hip -- y[M,N] = bf16(x[M,K] . W[K,N]) on the gfx950 matrix cores.
//
// Reduction schedule of the batch-invariant entry point (fixed by K alone):
//   K-block  = 32 = one v_mfma_f32_16x16x32_bf16,
//   segment  = KC = 512 consecutive K (16 blocks), accumulated from +0,
//   segments folded left to right 0..S-1 with fp32 adds, S = ceil(K/KC),
//   one round-to-nearest-even narrowing to bf16.
// This is the two-stage deterministic reduction of the Determinism article
// (section 4): per-slice partial sums written to a fixed workspace and added
// in the fixed index order, with no float atomics anywhere; the K split is
// the same whatever M is, and the M tile is padded rather than re-chosen.
//
// Two kernels implement that schedule; which one runs depends on M, and the
// bits never do (both issue the same matrix-core instruction on the same
// operands in the same order, start every segment from +0, and fold the
// segments with the same fp32 adds):
//   gemm_split_kernel  small M (weight streaming, HBM bound): one workgroup
//                      per (64-column tile, segment, 64-row tile); segment
//                      sums go to an fp32 workspace; the last workgroup of a
//                      tile to arrive (integer ticket) folds them in order.
//   gemm_tile_kernel   large M (matrix-core bound): 128x128 output tiles, all
//                      segments of K in one workgroup, folded in registers.
// Padding rows (>= M) load as zero, are never stored, and 16-row sub-tiles
// that are entirely padding skip their matrix-core ops.
//
// W is [K,N] row-major (N contiguous), while the matrix core wants 8
// consecutive K per lane for the B operand.  W tiles are therefore staged in
// LDS as they sit in memory and read back with the LDS transpose read
// (ds_read_b64_tr_b16), which hands each lane one column.
//
// The fast twin reuses both kernels with a schedule picked from M and the CU
// count: the split kernel with a K slice sized to fill the chip, and the tile
// kernel with a single accumulation chain over all of K (no segments).
#include "bi_common.h"
#include "bi_internal.h"

namespace bi {

static constexpr int KB = 32;        // K per matrix-core op
static constexpr int SPLIT_BN = 64;  // columns per split workgroup (4 waves x 16)
static constexpr int SPLIT_BM = 64;  // rows per split workgroup (4 sub-tiles of 16)
static constexpr int SPLIT_SK = 128; // K rows of W staged per LDS buffer
static constexpr int SPLIT_LDW = SPLIT_BN + 16;  // padded LDS row (elements)

// ---------------------------------------------------------------------------
// Split kernel (small M)
// ---------------------------------------------------------------------------
// grid = (N/64, S, ceil(M/64)), block = 256 (4 waves).  Wave w owns columns
// n0 + 16w .. +15 of the tile and every 16-row sub-tile that holds a row < M.
// Per stage of 128 K: the W slab (128 x 64) goes through LDS, the x
// fragments stay in registers; the next stage is fetched while this one runs.
// MAXSUB = 1 for M <= 16 (fewer registers), 4 otherwise.
template <int MAXSUB>
__global__ __launch_bounds__(256) void gemm_split_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W,
    float* __restrict__ part, int M, int N, int K, int KC) {
  __shared__ __attribute__((aligned(16))) uint16_t wl[2][SPLIT_SK * SPLIT_LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ntile = blockIdx.x;
  const int seg = blockIdx.y;
  const int mtile = blockIdx.z;
  const int n0 = ntile * SPLIT_BN;
  const int m0 = mtile * SPLIT_BM;
  const int k_begin = seg * KC;
  const int k_end = min(K, k_begin + KC);
  const int rows = min(SPLIT_BM, M - m0);
  const int nsub = min(MAXSUB, (rows + 15) >> 4);  // 16-row sub-tiles holding a real row

  // A operand lanes: row m0 + 16*sub + lane%16, k = kb + (lane/16)*8 .. +7.
  const int arow = lane & 15;
  const int g = lane >> 4;
  // B operand via transpose read: lane 4r+c of group g addresses row
  // kb + 8g + 4h + r, columns 16*wave + 4c .. +3, for h = 0, 1.
  const int tr_r = (lane & 15) >> 2;
  const int tr_c = lane & 3;

  u32x4_t wreg[4];
  u32x4_t acur[MAXSUB][4], anext[MAXSUB][4];
  // One stage: W rows k0..k0+127 (chunk c = tid + 256 i: row c/8, columns
  // 8*(c%8)..+7) and the x fragments of its four K-blocks.
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int k = k0 + (c >> 3);
      wreg[i] = (k < k_end) ? ldg128(W + (size_t)k * N + n0 + (c & 7) * 8)
                            : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int s = 0; s < MAXSUB; ++s) {
      const int m = m0 + s * 16 + arow;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kb = k0 + j * KB;
        anext[s][j] = (s < nsub && m < M && kb < k_end) ? ldg128(x + (size_t)m * K + kb + g * 8)
                                                         : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_w = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *(u32x4_t*)&wl[buf][(c >> 3) * SPLIT_LDW + (c & 7) * 8] = wreg[i];
    }
  };

  f32x4_t acc[MAXSUB];
#pragma unroll
  for (int s = 0; s < MAXSUB; ++s) acc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nstage = (k_end - k_begin + SPLIT_SK - 1) / SPLIT_SK;
  load_stage(k_begin);
  store_w(0);
#pragma unroll
  for (int s = 0; s < MAXSUB; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) acur[s][j] = anext[s][j];
  __syncthreads();
  for (int st = 0; st < nstage; ++st) {
    const int k0 = k_begin + st * SPLIT_SK;
    if (st + 1 < nstage) load_stage(k0 + SPLIT_SK);
    const uint16_t* wb = wl[st & 1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (k0 + j * KB < k_end) {
        const uint16_t* base = wb + (j * KB + 8 * g + tr_r) * SPLIT_LDW + 16 * wave + 4 * tr_c;
        const u32x2_t b0 = lds_read_tr16(base);
        const u32x2_t b1 = lds_read_tr16(base + 4 * SPLIT_LDW);
        const u32x4_t bfrag = u32x4_t{b0.x, b0.y, b1.x, b1.y};
#pragma unroll
        for (int s = 0; s < MAXSUB; ++s)
          if (s < nsub) acc[s] = mfma16x16x32(acur[s][j], bfrag, acc[s]);
      }
    }
    if (st + 1 < nstage) {
      store_w((st + 1) & 1);
#pragma unroll
      for (int s = 0; s < MAXSUB; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) acur[s][j] = anext[s][j];
    }
    __syncthreads();
  }

  // Segment partial -> workspace part[seg][m][n] (rows < M only).
  const int ccol = n0 + 16 * wave + (lane & 15);
#pragma unroll
  for (int s = 0; s < MAXSUB; ++s) {
    if (s < nsub) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + s * 16 + g * 4 + e;
        if (m < M) part[((size_t)seg * M + m) * N + ccol] = acc[s][e];
      }
    }
  }

}

// ---------------------------------------------------------------------------
// Skinny kernel (M <= 16, the decode regime: W streamed once, HBM bound)
// ---------------------------------------------------------------------------
// One workgroup of 512 lanes owns a 64-column tile of y (128-byte rows of W,
// so every W line fetched is used whole) and either
//   ALLK = false: one 512-row segment of K; its sum goes to the workspace and
//                 gemm_fold_kernel adds the segments in order afterwards, or
//   ALLK = true:  every segment of K in order, folded in registers, y written
//                 directly (used when the 64-column tiles alone fill the chip).
// The whole 64 KB W slab of a segment is requested at once (8 loads of 16 B
// per lane) and the next segment's slab is in flight while the current one
// is multiplied.  The slab sits in LDS with its 16-byte chunks XOR-swizzled
// by row, so the transpose reads of four consecutive rows hit distinct banks.
// Waves 0..3 each own one 16-column sub-tile; x fragments come straight from
// memory (rows >= M read as zero through the buffer range check).
static constexpr int SK_BN = 64;
static constexpr int SK_ROWS = 512;  // = KC

__device__ __forceinline__ int sk_phys(int row, int chunk) {  // element offset of a 16-B chunk
  return row * SK_BN + ((chunk ^ (row & 7)) << 3);
}

template <bool ALLK>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, uint16_t* __restrict__ y,
    float* __restrict__ part, int M, int N, int K, int S) {
  __shared__ __attribute__((aligned(16))) uint16_t wl[SK_ROWS * SK_BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int arow = lane & 15;
  const int tr_r = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int n0 = blockIdx.x * SK_BN;
  const int seg_begin = ALLK ? 0 : (int)blockIdx.y;
  const int seg_end = ALLK ? S : (int)blockIdx.y + 1;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)((size_t)K * N * 2));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
  const uint32_t row_bytes = (uint32_t)N * 2;

  // W slab of one segment: chunk c = tid + 512 i is row c/8, 16-B chunk c%8.
  u32x4_t wreg[8];
  auto issue_w = [&](int seg, bool valid) {
    uint32_t off = (uint32_t)(seg * SK_ROWS + (tid >> 3)) * row_bytes +
                   (uint32_t)(n0 + (tid & 7) * 8) * 2;
    if (!valid) off = 0x80000000u;  // past the end: zeros, no memory traffic
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wreg[i] = bufld128(wr, off);
      off = valid ? off + 64 * row_bytes : off;
    }
  };
  u32x4_t xc[16];
  auto issue_x = [&](int seg) {
    const uint32_t off = (uint32_t)(arow * K + seg * SK_ROWS + g * 8) * 2;
#pragma unroll
    for (int j = 0; j < 16; ++j) xc[j] = bufld128(xr, off + j * KB * 2);
  };

  f32x4_t tot = f32x4_t{0.f, 0.f, 0.f, 0.f};
  issue_w(seg_begin, true);
  for (int seg = seg_begin; seg < seg_end; ++seg) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + 512 * i;
      *(u32x4_t*)&wl[sk_phys(c >> 3, c & 7)] = wreg[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (wave < 4) issue_x(seg);
    issue_w(seg + 1, seg + 1 < seg_end);
    if (wave < 4) {
      const int nkb = min(SK_ROWS, K - seg * SK_ROWS) / KB;
      const int chunk = 2 * wave + (tr_c >> 1);
      const int sub = (tr_c & 1) * 4;
      f32x4_t a = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 16; ++kb) {
        if (kb < nkb) {
          const int r0 = kb * KB + 8 * g + tr_r;
          const u32x2_t b0 = lds_read_tr16(&wl[sk_phys(r0, chunk) + sub]);
          const u32x2_t b1 = lds_read_tr16(&wl[sk_phys(r0 + 4, chunk) + sub]);
          a = mfma16x16x32(xc[kb], u32x4_t{b0.x, b0.y, b1.x, b1.y}, a);
        }
      }
      const int col = n0 + 16 * wave + arow;
      if (ALLK) {
        if (seg == 0)
          tot = a;
        else
          tot = tot + a;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = g * 4 + e;
          if (m < M) part[((size_t)seg * M + m) * N + col] = a[e];
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  }
  if (ALLK && wave < 4) {
    const int col = n0 + 16 * wave + arow;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = g * 4 + e;
      if (m < M) y[(size_t)m * N + col] = (uint16_t)f32_to_bf16_bits(tot[e]);
    }
  }
}

// Ordered fold of segment sums: y = bf16(((p0 + p1) + p2) + ...), fp32.
// One lane per (row, 4 columns); every segment's load is issued before the
// adds.  grid = (ceil(N/256), M), block = 64.
__global__ __launch_bounds__(64) void gemm_fold_kernel(const float* __restrict__ part,
                                                       uint16_t* __restrict__ y, int M, int N,
                                                       int S) {
  const int c4 = blockIdx.x * 64 + threadIdx.x;
  const int m = blockIdx.y;
  if (c4 * 4 >= N) return;
  const f32x4_t* p = (const f32x4_t*)(part + (size_t)m * N) + c4;
  const size_t step = (size_t)M * N / 4;
  f32x4_t acc = p[0];
  for (int s0 = 1; s0 < S; s0 += 8) {
    f32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) v[u] = p[(size_t)(s0 + u) * step];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) acc = acc + v[u];
  }
  uint32_t* out = (uint32_t*)(y + (size_t)m * N + c4 * 4);
  out[0] = pack_bf16x2(acc[0], acc[1]);
  out[1] = pack_bf16x2(acc[2], acc[3]);
}

// ---------------------------------------------------------------------------
// Tile kernel (large M)
// ---------------------------------------------------------------------------
static constexpr int TBM = 128, TBN = 128, TBK = 64;
static constexpr int T_LDX = TBK + 8;    // padded x row in LDS (elements)
static constexpr int T_LDW = TBN + 16;   // padded W row in LDS (elements)

// grid = (N/128, ceil(M/128)), block = 256: waves in a 2x2 grid, 64x64 each.
// FOLD: true  -> segments of KC from +0, folded in registers (invariant);
//       false -> one accumulation chain over all of K (fast twin).
template <bool FOLD>
__global__ __launch_bounds__(256) void gemm_tile_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, uint16_t* __restrict__ y,
    int M, int N, int K, int KC) {
  __shared__ __attribute__((aligned(16))) uint16_t xl[2][TBM * T_LDX];
  __shared__ __attribute__((aligned(16))) uint16_t wl[2][TBK * T_LDW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * TBN;
  const int m0 = blockIdx.y * TBM;

  // Loaders: x stage 128 rows x 64 K (8 chunks per row), W stage 64 rows x
  // 128 columns (16 chunks per row); 4 chunks of 16 B per thread for each.
  u32x4_t xr[4], wr[4];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, kc = c & 7;
      const int m = m0 + r;
      if (m < M && k0 + kc * 8 < K)
        xr[i] = ldg128(x + (size_t)m * K + k0 + kc * 8);
      else
        xr[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 4, nc = c & 15;
      const int k = k0 + r;
      if (k < K && n0 + nc * 8 < N)
        wr[i] = ldg128(W + (size_t)k * N + n0 + nc * 8);
      else
        wr[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *(u32x4_t*)&xl[buf][(c >> 3) * T_LDX + (c & 7) * 8] = xr[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      *(u32x4_t*)&wl[buf][(c >> 4) * T_LDW + (c & 15) * 8] = wr[i];
    }
  };

  f32x4_t acc[4][4];
  f32x4_t tot[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      tot[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  // 16-row sub-tiles of this wave that hold at least one row < M.
  const int wrow0 = m0 + wm * 64;
  const int nsub = max(0, min(4, (M - wrow0 + 15) >> 4));

  const int g = lane >> 4;
  const int tr_r = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int arow = lane & 15;

  const int nstage = (K + TBK - 1) / TBK;
  const int blocks_per_seg = KC / KB;
  int seg = 0;
  int kblk_in_seg = 0;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nstage; ++st) {
    const int k0 = st * TBK;
    if (st + 1 < nstage) load_stage(k0 + TBK);
    const uint16_t* xs = xl[st & 1];
    const uint16_t* ws = wl[st & 1];
    const int nkb = min(TBK, K - k0) / KB;
    for (int j = 0; j < nkb; ++j) {
      u32x4_t bf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint16_t* base = ws + (j * KB + 8 * g + tr_r) * T_LDW + wn * 64 + t * 16 + 4 * tr_c;
        const u32x2_t b0 = lds_read_tr16(base);
        const u32x2_t b1 = lds_read_tr16(base + 4 * T_LDW);
        bf[t] = u32x4_t{b0.x, b0.y, b1.x, b1.y};
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < nsub) {
          const u32x4_t af =
              *(const u32x4_t*)&xs[(wm * 64 + s * 16 + arow) * T_LDX + j * KB + g * 8];
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[s][t] = mfma16x16x32(af, bf[t], acc[s][t]);
        }
      }
      if (FOLD) {
        // segment boundary: fold this segment's sum into the running total
        if (++kblk_in_seg == blocks_per_seg || (k0 + (j + 1) * KB) >= K) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              if (seg == 0)
                tot[s][t] = acc[s][t];
              else
                tot[s][t] = tot[s][t] + acc[s][t];
              acc[s][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
          ++seg;
          kblk_in_seg = 0;
        }
      }
    }
    if (st + 1 < nstage) store_stage((st + 1) & 1);
    __syncthreads();
  }

  // Epilogue: narrow and store rows < M.
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < nsub) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int col = n0 + wn * 64 + t * 16 + (lane & 15);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = wrow0 + s * 16 + (lane >> 4) * 4 + e;
          const float v = FOLD ? tot[s][t][e] : acc[s][t][e];
          if (m < M && col < N) y[(size_t)m * N + col] = (uint16_t)f32_to_bf16_bits(v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tile kernel v3 (large M, matrix-core bound)
// ---------------------------------------------------------------------------
// 256 x 128 output tile per workgroup of 8 waves (4 x 2), each wave 64 x 64
// (4 x 4 matrix-core tiles), two waves per SIMD.  K advances in stages of 64
// (two K-blocks): the next stage's x slab (256 x 64) and W slab (64 x 128)
// are fetched into registers while the current stage is multiplied out of
// LDS, then written to the other of two LDS stage buffers.  LDS rows are
// XOR-swizzled in 16-byte chunks so that the A-operand reads (8 rows at a
// time) and the transpose reads of W (4 rows at a time) hit distinct banks.
// FOLD: segments of KC from +0 folded in order in registers (batch-invariant
// schedule); without FOLD one accumulation chain runs over all of K.
// Workgroups are mapped to tiles so that each XCD (workgroups are dispatched
// to the 8 XCDs round robin) works on a contiguous band of tiles, m fastest:
// workgroups sharing an L2 share W column panels and x row panels.
static constexpr int T2_BN = 128, T2_BK = 64;
static constexpr int T2_WS = T2_BK * T2_BN;          // W slab elements (16 KB)

// element offset of logical 16-B chunk `c` of row `r` in the x slab (8 chunks per row)
__device__ __forceinline__ int t2_xphys(int r, int c) { return r * T2_BK + ((c ^ (r & 7)) << 3); }
// element offset of logical 16-B chunk `c` of k-row `r` in the W slab (16 chunks
// per row), which follows an x slab of `xs` elements
__device__ __forceinline__ int t2_wphys(int xs, int r, int c) {
  return xs + r * T2_BN + ((c ^ ((r & 3) << 1)) << 3);
}

// BM rows per workgroup, 2*BM lanes (BM/64 x 2 waves of 64 x 64).  256 is the
// size in use: with the fold's second set of accumulators, 128 spills.
// SLICE: the workgroup covers only K slice blockIdx.y ([y*KC, y*KC + KC)),
// accumulated in one chain from +0, and writes the fp32 slice sum to
// part[y][M][N] for gemm_fold_kernel (used when the tiles alone are too few
// to fill the chip; with KC = 512 the slice is exactly one segment).
template <bool FOLD, int BM, bool SLICE = false>
__global__ __launch_bounds__(BM * 2, 2) void gemm_tile2_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, uint16_t* __restrict__ y,
    int M, int N, int K, int KC, int tm, int tn, int remap, float* __restrict__ part = nullptr) {
  constexpr int NT = BM * 2;                  // lanes per workgroup
  constexpr int T2_BM = BM;
  constexpr int T2_XS = BM * T2_BK;           // x slab elements
  constexpr int T2_STAGE = T2_XS + T2_WS;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][T2_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int tr_r = l16 >> 2, tr_c = lane & 3;

  int t = blockIdx.x;
  if (remap) t = (t & 7) * ((tm * tn) >> 3) + (t >> 3);
  const int m0 = (t % tm) * T2_BM;
  const int n0 = (t / tm) * T2_BN;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)((size_t)K * N * 2));
  // K range of this workgroup: all of K, or one slice
  const int kbeg = SLICE ? (int)blockIdx.y * KC : 0;
  const int kend = SLICE ? min(K, kbeg + KC) : K;

  // Loads of one stage: x chunks c = tid + NT i (row c/8, chunk c%8), W
  // chunks c = tid + NT i (k-row c/16, chunk c%16).  Rows >= M and k >= K
  // read as zero through the buffer range check.
  constexpr int XL = T2_XS / 8 / NT;          // 16-B x chunks per lane per stage (4)
  constexpr int WL = T2_WS / 8 / NT;          // 16-B W chunks per lane per stage (2 or 4)
  const uint32_t xoff0 = (uint32_t)((m0 + (tid >> 3)) * K + (tid & 7) * 8) * 2;
  const uint32_t xrowstep = (uint32_t)K * 2 * (NT / 8);    // NT/8 rows of x, in bytes
  const uint32_t woff0 = (uint32_t)((tid >> 4) * N + n0 + (tid & 15) * 8) * 2;
  const uint32_t wrowstep = (uint32_t)N * 2 * (NT / 16);   // NT/16 k-rows of W, in bytes
  u32x4_t xs[XL], ws[WL];
  auto load_stage = [&](int k0) {
    const bool valid = k0 < kend;   // past the end: zeros, no memory traffic
#pragma unroll
    for (int i = 0; i < XL; ++i)
      xs[i] = bufld128(xr, valid ? xoff0 + i * xrowstep + (uint32_t)k0 * 2 : 0x80000000u);
#pragma unroll
    for (int i = 0; i < WL; ++i)
      ws[i] = bufld128(wr, valid ? woff0 + i * wrowstep + (uint32_t)k0 * N * 2 : 0x80000000u);
  };
  auto store_stage = [&](uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int c = tid + NT * i;
      *(u32x4_t*)(buf + t2_xphys(c >> 3, c & 7)) = xs[i];
    }
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int c = tid + NT * i;
      *(u32x4_t*)(buf + t2_wphys(T2_XS, c >> 4, c & 15)) = ws[i];
    }
  };

  f32x4_t acc[4][4];
  f32x4_t tot[FOLD ? 4 : 1][FOLD ? 4 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (FOLD ? 4 : 1); ++i)
#pragma unroll
    for (int j = 0; j < (FOLD ? 4 : 1); ++j) tot[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wrow0 = m0 + wm * 64;
  const int nsub = max(0, min(4, (M - wrow0 + 15) >> 4));
  const int blocks_per_seg = KC / KB;
  int kblk = 0;  // K-blocks done in the current segment
  int seg = 0;

  // LDS element offsets of this lane's operand reads for K-block 0 of a
  // stage; sub-tile s adds 16 rows (the x swizzle uses row % 8, unchanged),
  // K-block 1 adds 4 chunks (x) or 32 rows (W, swizzle uses row % 4).
  int aoff[2], boff[4][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) aoff[j] = t2_xphys(wm * 64 + l16, j * 4 + g);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int col = wn * 64 + tt * 16 + 4 * tr_c;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      boff[tt][h] = t2_wphys(T2_XS, 8 * g + 4 * h + tr_r, col >> 3) + (col & 7);
  }

  // operand fragments of one K-block: A for the 4 sub-tiles, B for the 4 columns
  u32x4_t af[2][4], bf[2][4];
  auto read_frags = [&](const uint16_t* buf, int j, int set) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const u32x2_t b0 = lds_read_tr16(buf + boff[tt][0] + j * KB * T2_BN);
      const u32x2_t b1 = lds_read_tr16(buf + boff[tt][1] + j * KB * T2_BN);
      bf[set][tt] = u32x4_t{b0.x, b0.y, b1.x, b1.y};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      af[set][s] = *(const u32x4_t*)(buf + aoff[j] + s * 16 * T2_BK);
  };
  auto fold_if_segment_end = [&](int kdone) {
    if (FOLD) {
      if (++kblk == blocks_per_seg || kdone >= kend) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            if (seg == 0)
              tot[s][tt] = acc[s][tt];
            else
              tot[s][tt] = tot[s][tt] + acc[s][tt];
            acc[s][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
        ++seg;
        kblk = 0;
      }
    }
  };
  // Multiply one stage: the fragments of K-block 1 are read while the
  // multiplies of K-block 0 run.  Every 16-row sub-tile is multiplied,
  // padding rows included (they hold zeros and are never stored).
  auto compute = [&](const uint16_t* buf, int k0) {
    read_frags(buf, 0, 0);
    const bool two = k0 + KB < kend;
    if (two) read_frags(buf, 1, 1);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) acc[s][tt] = mfma16x16x32(af[0][s], bf[0][tt], acc[s][tt]);
    fold_if_segment_end(k0 + KB);
    if (two) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[s][tt] = mfma16x16x32(af[1][s], bf[1][tt], acc[s][tt]);
      fold_if_segment_end(k0 + 2 * KB);
    }
  };
  auto lds_barrier = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };

  const int nstage = (kend - kbeg + T2_BK - 1) / T2_BK;
  load_stage(kbeg);
  store_stage(lds[0]);
  lds_barrier();
  for (int st = 0; st < nstage; ++st) {
    load_stage(kbeg + (st + 1) * T2_BK);
    compute(lds[st & 1], kbeg + st * T2_BK);
    if (st + 1 < nstage) store_stage(lds[(st + 1) & 1]);
    lds_barrier();
  }

#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s < nsub) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int col = n0 + wn * 64 + tt * 16 + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = wrow0 + s * 16 + g * 4 + e;
          const float v = FOLD ? tot[s][tt][e] : acc[s][tt][e];
          if (m < M && col < N) {
            if (SLICE)
              part[((size_t)blockIdx.y * M + m) * N + col] = v;
            else
              y[(size_t)m * N + col] = (uint16_t)f32_to_bf16_bits(v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static constexpr int BI_KC = 512;  // invariant segment length
static constexpr int TILE_BM = 256;  // rows per tile-kernel workgroup (8 waves)
static constexpr int SPLIT_MAX_M = 64;
static constexpr int SKINNY_MAX_M = 16;
static constexpr int SKINNY_ALLK_TILES = 256;  // 64-column tiles that fill the chip alone

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Which kernels run for (M, N, K).  The bits never depend on it.
static constexpr int TILE_MIN_TILES = 192;  // fewer tiles than this: split K into slices

enum class GemmPath { Tile, TileSlice, SkinnyAllK, SkinnySeg, Split };
static GemmPath gemm_path(int64_t M, int64_t N) {
  if (M > SPLIT_MAX_M)
    return ceil_div(M, TILE_BM) * ceil_div(N, T2_BN) >= TILE_MIN_TILES ? GemmPath::Tile
                                                                         : GemmPath::TileSlice;
  if (M <= SKINNY_MAX_M) return (N / SK_BN >= SKINNY_ALLK_TILES) ? GemmPath::SkinnyAllK
                                                                  : GemmPath::SkinnySeg;
  return GemmPath::Split;
}

// K slice of the tile kernel: the invariant schedule always uses 512 (one
// segment per slice); the fast twin uses as few slices as fill the chip.
// At M <= 64 the fast twin keeps the invariant kernels (their schedule is
// already the fastest layout for streaming W).
int64_t fast_split_kc(int64_t M, int64_t N, int64_t K, int num_cus) {
  const int64_t tiles = ceil_div(M, TILE_BM) * ceil_div(N, T2_BN);
  const int64_t slices = std::max<int64_t>(1, ceil_div(std::max(num_cus, 1), tiles));
  return ceil_div(ceil_div(K, slices), T2_BK) * T2_BK;
}
static int64_t slice_kc(int64_t M, int64_t N, int64_t K, bool fast, int num_cus) {
  return fast ? fast_split_kc(M, N, K, num_cus) : BI_KC;
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, bool fast, int num_cus) {
  const GemmPath p = gemm_path(M, N);
  if (p == GemmPath::Tile || p == GemmPath::SkinnyAllK) return 0;
  const int64_t kc = p == GemmPath::TileSlice ? slice_kc(M, N, K, fast, num_cus) : BI_KC;
  return (size_t)ceil_div(K, kc) * (size_t)M * (size_t)N * sizeof(float);
}

int launch_gemm(const uint16_t* x, const uint16_t* W, uint16_t* y, int64_t M, int64_t N,
                int64_t K, void* ws, size_t ws_bytes, hipStream_t stream, bool fast, int num_cus) {
  const int64_t S = ceil_div(K, BI_KC);
  const GemmPath p = gemm_path(M, N);
  if (p == GemmPath::Tile) {
    constexpr int BM = TILE_BM;
    const int64_t tm = ceil_div(M, BM), tn = ceil_div(N, T2_BN);
    const int remap = ((tm * tn) % 8 == 0) ? 1 : 0;
    dim3 grid((unsigned)(tm * tn));
    if (fast)
      hipLaunchKernelGGL((gemm_tile2_kernel<false, BM>), grid, dim3(2 * BM), 0, stream, x, W, y,
                         (int)M, (int)N, (int)K, (int)K, (int)tm, (int)tn, remap);
    else
      hipLaunchKernelGGL((gemm_tile2_kernel<true, BM>), grid, dim3(2 * BM), 0, stream, x, W, y,
                         (int)M, (int)N, (int)K, BI_KC, (int)tm, (int)tn, remap);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
  }
  if (p == GemmPath::TileSlice) {
    constexpr int BM = TILE_BM;
    const int64_t kc = slice_kc(M, N, K, fast, num_cus);
    const int64_t ns = ceil_div(K, kc);
    const int64_t tm = ceil_div(M, BM), tn = ceil_div(N, T2_BN);
    if (ns > 65535) return BI_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < (size_t)ns * (size_t)M * (size_t)N * sizeof(float)) return BI_ERR_WORKSPACE;
    float* part = (float*)ws;
    const int remap = ((tm * tn) % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((gemm_tile2_kernel<false, BM, true>), dim3((unsigned)(tm * tn), (unsigned)ns),
                       dim3(2 * BM), 0, stream, x, W, y, (int)M, (int)N, (int)K, (int)kc, (int)tm,
                       (int)tn, remap, part);
    if (hipGetLastError() != hipSuccess) return BI_ERR_HIP;
    hipLaunchKernelGGL(gemm_fold_kernel, dim3((unsigned)ceil_div(N, 256), (unsigned)M), dim3(64),
                       0, stream, part, y, (int)M, (int)N, (int)ns);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
  }
  if (p == GemmPath::SkinnyAllK) {
    hipLaunchKernelGGL(gemm_skinny_kernel<true>, dim3((unsigned)(N / SK_BN), 1), dim3(512), 0,
                       stream, x, W, y, (float*)nullptr, (int)M, (int)N, (int)K, (int)S);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
  }
  if (S > 65535) return BI_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < (size_t)S * (size_t)M * (size_t)N * sizeof(float)) return BI_ERR_WORKSPACE;
  float* part = (float*)ws;
  if (p == GemmPath::SkinnySeg) {
    hipLaunchKernelGGL(gemm_skinny_kernel<false>, dim3((unsigned)(N / SK_BN), (unsigned)S),
                       dim3(512), 0, stream, x, W, y, part, (int)M, (int)N, (int)K, (int)S);
  } else {
    dim3 grid((unsigned)(N / SPLIT_BN), (unsigned)S, (unsigned)ceil_div(M, SPLIT_BM));
    hipLaunchKernelGGL(gemm_split_kernel<4>, grid, dim3(256), 0, stream, x, W, part, (int)M,
                       (int)N, (int)K, BI_KC);
  }
  if (hipGetLastError() != hipSuccess) return BI_ERR_HIP;
  hipLaunchKernelGGL(gemm_fold_kernel, dim3((unsigned)ceil_div(N, 256), (unsigned)M), dim3(64),
                     0, stream, part, y, (int)M, (int)N, (int)S);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi
