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
// Several kernels implement that schedule; which ones run depends on (M, N),
// and the bits never do (all issue the same matrix-core instruction on the
// same operands in the same order, start every segment from +0, and fold the
// segments with the same fp32 adds in index order):
//   gemm_skinny_kernel  M <= 16 (weight streaming, HBM bound): one 512-lane
//                       workgroup per 64-column tile; with enough tiles to
//                       fill the chip it streams all segments and folds them
//                       in registers, otherwise one workgroup per (tile,
//                       segment) writes the segment sum to the workspace.
//   gemm_split_kernel   16 < M <= 64: one workgroup per (64-column tile,
//                       segment, 64-row tile), segment sums to the workspace.
//   gemm_fold_kernel    adds workspace segment sums in index order, narrows.
//   gemm_tile_kernel    M > 64 (matrix-core bound): 256x128 output tiles, all
//                       segments folded in registers; with too few tiles to
//                       fill the chip, one workgroup per (tile, segment)
//                       writes segment sums for gemm_fold_kernel instead.
// Padding rows (>= M) load as zero through the buffer range check and are
// never stored.
//
// W is [K,N] row-major (N contiguous), while the matrix core wants 8
// consecutive K per lane for the B operand.  W tiles are therefore staged in
// LDS as they sit in memory and read back with the LDS transpose read
// (ds_read_b64_tr_b16), which hands each lane one column.
//
// The fast twin reuses these kernels with a schedule picked from M and the
// CU count: at M > 64 the tile kernel runs one accumulation chain over all of
// K (no segments), sliced in K only as far as needed to fill the chip; at
// M <= 64 it runs the invariant kernels unchanged.
#include <type_traits>

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
// Tile kernel (large M, matrix-core bound)
// ---------------------------------------------------------------------------
// 256 x 128 output tile per workgroup of 8 waves (4 x 2), each wave 64 x 64
// (4 x 4 matrix-core tiles), two waves per SIMD.  K advances in stages of 64
// (two K-blocks) through a ring of three LDS stage buffers (48 KB each) that
// direct-to-LDS buffer loads fill three stages ahead; one barrier per stage.
// Fragments are read one K-block ahead, across stage boundaries.
//
// LDS layout of a stage: the x slab (256 rows x 64 k, 128 B rows) then the W
// slab (64 k-rows x 128 columns, 256 B rows), both in 16-B chunks whose index
// is XORed with low row bits, so that the A-operand reads (16 rows, one chunk
// each) and the transpose reads of W (16 k-rows, 32 B each) spread over all
// LDS banks.  A direct-to-LDS load writes lane i at 16 i, so each lane
// fetches the global chunk whose swizzled home is its slot.
//
// Each 16x16 product is issued as y^T = W^T x^T (W fragment as the A operand):
// the same products in the same order as x W, with the accumulator holding
// four consecutive columns of one row per lane, which makes the stores 8 B.
//
// FOLD: segments of KC (a multiple of 64) from +0, folded in order into the
// running total after each (batch-invariant schedule); the first K-block of
// a segment is issued with a zero accumulator.  Without FOLD, one chain runs
// over the workgroup's K range.  SLICE: the workgroup covers only K slice
// blockIdx.y ([y*KC, y*KC + KC)) and writes its fp32 sum to part[y][M][N].
//
// Workgroups are dispatched to the 8 XCDs round robin.  remap 2 gives each
// XCD a band of whole tile columns, walked in groups of 4 tile rows, so that
// the 32 workgroups an XCD runs at once share 4 x panels and 8 W panels in
// its L2; remap 1 gives each XCD a contiguous band of tiles, m fastest.
static constexpr int TL_BM = 256, TL_BN = 128, TL_BK = 64;
static constexpr int TL_XS = TL_BM * TL_BK;             // x slab elements (32 KB)
static constexpr int TL_STAGE = TL_XS + TL_BK * TL_BN;  // + W slab (16 KB)

__device__ __forceinline__ int tl_xphys(int r, int c) { return r * TL_BK + ((c ^ (r & 7)) << 3); }
__device__ __forceinline__ int tl_wswz(int r) { return ((r & 3) << 1) ^ (((r >> 3) & 1) << 3); }
__device__ __forceinline__ int tl_wphys(int r, int c) {
  return TL_XS + r * TL_BN + ((c ^ tl_wswz(r)) << 3);
}

template <bool FOLD, bool SLICE>
__global__ __launch_bounds__(512, 2) void gemm_tile_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, uint16_t* __restrict__ y,
    int M, int N, int K, int KC, int tm, int tn, int remap, float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[3 * TL_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int tr_r = l16 >> 2, tr_c = lane & 3;

  int t = blockIdx.x;
  if (remap == 1) {
    t = (t & 7) * ((tm * tn) >> 3) + (t >> 3);
  } else if (remap == 2) {
    const int ncols = tn >> 3, xcd = t & 7, i = t >> 3;
    const int first = (i / (4 * ncols)) * 4, gm = min(4, tm - first);
    const int r = i - first * ncols;
    t = (xcd * ncols + r / gm) * tm + first + r % gm;
  }
  const int m0 = (t % tm) * TL_BM;
  const int n0 = (t / tm) * TL_BN;

  const i32x4_t xr = make_rsrc_words(x, (uint32_t)((size_t)M * K * 2));
  const i32x4_t wr = make_rsrc_words(W, (uint32_t)((size_t)K * N * 2));
  const int kbeg = SLICE ? (int)blockIdx.y * KC : 0;
  const int kend = SLICE ? min(K, kbeg + KC) : K;
  const int nstage = (kend - kbeg + TL_BK - 1) / TL_BK;

  // Each wave instruction fills 1 KB of a stage: wave w fills x regions
  // 4w..4w+3 (8 rows each) and W regions 2w, 2w+1 (4 k-rows each).
  uint32_t xoff[4], woff[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = (wave * 4 + i) * 64 + lane;
    const int r = p >> 3, c = (p & 7) ^ (r & 7);
    xoff[i] = ((uint32_t)(m0 + r) * (uint32_t)K + (uint32_t)(kbeg + c * 8)) * 2u;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = (wave * 2 + i) * 64 + lane;
    const int r = p >> 4, c = (p & 15) ^ tl_wswz(r);
    woff[i] = ((uint32_t)(kbeg + r) * (uint32_t)N + (uint32_t)(n0 + c * 8)) * 2u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(BI_LDS void*)lds;
  // Loads of stage st.  Past the last stage they take an offset outside the
  // buffer (zeros, no memory traffic), so every stage issues exactly six per
  // wave and the counter waits below hold.  Rows >= M and k >= K read as zero.
  auto dma = [&](int st) {
    const bool valid = st < nstage;
    const uint32_t base = lds0 + (uint32_t)((st % 3) * TL_STAGE * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      lds_dma16(xr, valid ? xoff[i] + (uint32_t)(st * TL_BK * 2) : 0x80000000u,
                base + (uint32_t)((wave * 4 + i) * 1024));
#pragma unroll
    for (int i = 0; i < 2; ++i)
      lds_dma16(wr, valid ? woff[i] + (uint32_t)(st * TL_BK) * (uint32_t)N * 2u : 0x80000000u,
                base + (uint32_t)(TL_XS * 2 + (wave * 2 + i) * 1024));
  };

  f32x4_t acc[4][4];
  f32x4_t tot[FOLD ? 4 : 1][FOLD ? 4 : 1];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // -0 + s == s exactly for every s, so the first fold copies the first
  // segment's sum bit for bit
#pragma unroll
  for (int i = 0; i < (FOLD ? 4 : 1); ++i)
#pragma unroll
    for (int j = 0; j < (FOLD ? 4 : 1); ++j) tot[i][j] = f32x4_t{-0.f, -0.f, -0.f, -0.f};

  // lane's element offsets within a stage (K-block 0)
  const int aoff = tl_xphys(wm * 64 + l16, g);
  int boff[4][2];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int col = wn * 64 + tt * 16 + 4 * tr_c;
#pragma unroll
    for (int h = 0; h < 2; ++h) boff[tt][h] = tl_wphys(8 * g + 4 * h + tr_r, col >> 3) + (col & 7);
  }

  u32x4_t af[2][4], bf[2][4];
  // fragments of K-block j (0 or 1) of stage st into set j
  auto read_frags = [&](int st, int j) {
    const uint16_t* buf = lds + (st % 3) * TL_STAGE;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const u32x2_t b0 = lds_read_tr16(buf + boff[tt][0] + j * KB * TL_BN);
      const u32x2_t b1 = lds_read_tr16(buf + boff[tt][1] + j * KB * TL_BN);
      bf[j][tt] = u32x4_t{b0.x, b0.y, b1.x, b1.y};
    }
    // K-block 1 is logical chunk g + 4 of the row: the swizzle keeps bit 2
#pragma unroll
    for (int s = 0; s < 4; ++s)
      af[j][s] = *(const u32x4_t*)(buf + (j ? (aoff ^ 32) : aoff) + s * 16 * TL_BK);
  };
  auto mma = [&](int j, bool from_zero) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
        acc[s][tt] = mfma16x16x32(bf[j][tt], af[j][s],
                                  from_zero ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[s][tt]);
  };
  auto fold = [&]() {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) tot[s][tt] = tot[s][tt] + acc[s][tt];
  };
  // One stage: K-block 0 (from +0 when it opens a segment), barrier, refill
  // of the buffer just consumed, next stage's K-block 0 fragments, K-block 1.
  auto stage = [&](int st, auto zero) {
    const bool two = kbeg + st * TL_BK + KB < kend;
    // read even when K-block 1 is past K (the fragments are then unused), so
    // that the LDS-counter waits see one path
    read_frags(st, 1);
    // K-block 0's fragments (the 12 LDS reads before these 12) have arrived
    __builtin_amdgcn_s_waitcnt(0xCC7F);  // lgkmcnt(12); vmcnt, expcnt unconstrained
    __builtin_amdgcn_sched_barrier(0);
    mma(0, decltype(zero)::value);
    __builtin_amdgcn_sched_barrier(0);
    // this wave's loads of stage st+1 have landed (only stage st+2's six may
    // be in flight) and its reads of stage st are done; after the barrier
    // every wave's are, so stage st's buffer can be refilled
    asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    dma(st + 3);
    read_frags(st + 1, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (two) mma(1, false);
  };

  dma(0);
  dma(1);
  dma(2);
  asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
  read_frags(0, 0);
  const int sps = FOLD ? KC / TL_BK : nstage;  // stages per segment
  int st = 0;
  for (;;) {
    stage(st, std::true_type{});
    const int seg_end = min(nstage, st + sps);
    for (++st; st < seg_end; ++st) stage(st, std::false_type{});
    if (st >= nstage) break;
    fold();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (FOLD) fold();

  const int wrow0 = m0 + wm * 64;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int m = wrow0 + s * 16 + l16;
    if (m < M && n0 + wn * 64 < N) {  // N is a multiple of 64: a wave's columns are all in or out
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f32x4_t v = FOLD ? tot[s][tt] : acc[s][tt];
        const int col = n0 + wn * 64 + tt * 16 + g * 4;
        if (SLICE) {
          *(f32x4_t*)&part[((size_t)blockIdx.y * M + m) * N + col] = v;
        } else {
          *(u32x2_t*)&y[(size_t)m * N + col] =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static constexpr int BI_KC = 512;  // invariant segment length
static constexpr int TILE_BM = TL_BM;  // rows per tile-kernel workgroup (8 waves)
static constexpr int SPLIT_MAX_M = 64;
static constexpr int SKINNY_MAX_M = 16;
static constexpr int SKINNY_ALLK_TILES = 256;  // 64-column tiles that fill the chip alone

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Which kernels run for (M, N, K).  The bits never depend on it.
static constexpr int TILE_MIN_TILES = 192;  // fewer tiles than this: split K into slices

enum class GemmPath { Tile, TileSlice, SkinnyAllK, SkinnySeg, Split };
static GemmPath gemm_path(int64_t M, int64_t N) {
  if (M > SPLIT_MAX_M)
    return ceil_div(M, TILE_BM) * ceil_div(N, TL_BN) >= TILE_MIN_TILES ? GemmPath::Tile
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
  const int64_t tiles = ceil_div(M, TILE_BM) * ceil_div(N, TL_BN);
  const int64_t slices = std::max<int64_t>(1, ceil_div(std::max(num_cus, 1), tiles));
  return ceil_div(ceil_div(K, slices), TL_BK) * TL_BK;
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
  if (p == GemmPath::Tile || p == GemmPath::TileSlice) {
    const int64_t tm = ceil_div(M, TILE_BM), tn = ceil_div(N, TL_BN);
    const int remap = (tn % 8 == 0) ? 2 : ((tm * tn) % 8 == 0) ? 1 : 0;
    if (p == GemmPath::Tile) {
      dim3 grid((unsigned)(tm * tn));
      if (fast)
        hipLaunchKernelGGL((gemm_tile_kernel<false, false>), grid, dim3(512), 0, stream, x, W, y,
                           (int)M, (int)N, (int)K, (int)K, (int)tm, (int)tn, remap, (float*)nullptr);
      else
        hipLaunchKernelGGL((gemm_tile_kernel<true, false>), grid, dim3(512), 0, stream, x, W, y,
                           (int)M, (int)N, (int)K, BI_KC, (int)tm, (int)tn, remap, (float*)nullptr);
      return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
    }
    const int64_t kc = slice_kc(M, N, K, fast, num_cus);
    const int64_t ns = ceil_div(K, kc);
    if (ns > 65535) return BI_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < (size_t)ns * (size_t)M * (size_t)N * sizeof(float)) return BI_ERR_WORKSPACE;
    float* part = (float*)ws;
    hipLaunchKernelGGL((gemm_tile_kernel<false, true>), dim3((unsigned)(tm * tn), (unsigned)ns),
                       dim3(512), 0, stream, x, W, y, (int)M, (int)N, (int)K, (int)kc, (int)tm,
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
