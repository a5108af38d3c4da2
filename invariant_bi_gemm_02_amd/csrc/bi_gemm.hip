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
// the same whatever M is.  The arithmetic unit of the schedule is a 16-row
// matrix-core sub-tile, padded with zero rows past M; how many sub-tiles
// one workgroup takes (16, 32, 64, 128 or 256 rows) and which kernel runs
// them follow M, which moves work between workgroups and never changes a bit.
//
// Several kernels implement that schedule; which ones run depends on (M, N),
// and the bits never do (all issue the same matrix-core instruction on the
// same operands in the same order, start every segment from +0, and fold the
// segments with the same fp32 adds in index order):
//   gemm_skinny_kernel  M <= 64 (weight streaming, HBM bound): one 512-lane
//                       workgroup per (128-column tile, segment) writes the
//                       segment sum to the workspace.
//   gemm_fold_kernel    adds workspace segment sums in index order, narrows.
//   gemm_tile_kernel    M > 64 (matrix-core bound): 256x128 output tiles, all
//                       segments folded in registers; with too few tiles to
//                       fill the chip, one workgroup per (tile, run of
//                       consecutive segments) writes each segment's sum for
//                       gemm_fold_kernel instead.
//   gemm_wide_kernel    other tile shapes on a ring of one K-block per stage:
//                       64x128, 128x128 and 256x192 with every segment
//                       folded in registers (where 256x128 tiles would leave
//                       CUs idle or a partial last round), 256x256 for the
//                       fast twin.
// Padding rows (>= M) load as zero through the buffer range check and are
// never stored.
//
// W is [K,N] row-major (N contiguous), while the matrix core wants 8
// consecutive K per lane for the B operand.  W tiles are therefore staged in
// LDS as they sit in memory and read back with the LDS transpose read
// (ds_read_b64_tr_b16), which hands each lane one column.
//
// The fast twin reuses these kernels with a schedule picked from M and the
// CU count: at M > 64 one accumulation chain over all of K (no segments), on
// 256x256 tiles where those fill the chip, else on 256x128 tiles sliced in K
// only as far as needed to fill it; at M <= 64 it runs the invariant kernels
// unchanged.
#include <type_traits>

#include "bi_common.h"
#include "bi_internal.h"

namespace bi {

static constexpr int KB = 32;        // K per matrix-core op

// ---------------------------------------------------------------------------
// Skinny kernel (M <= 64, the decode regime: W streamed once, HBM bound)
// ---------------------------------------------------------------------------
// One workgroup of 512 lanes per (BN-column tile, 512-row segment of K),
// BN = 128: 256-byte pieces of W rows, which the memory system streams
// faster than 128-byte ones.  The segment's sum goes to the workspace and
// gemm_fold_kernel adds the segments in order.  The x slab (16 MT rows,
// padded: rows >= M read as zero through the buffer range check) is
// requested first, then the whole W slab (16 B per lane per load, held in
// registers).  W passes through LDS a quarter at a time (128 rows): each
// quarter is written as soon as its loads land and its four K-blocks run
// while the later quarters are still in flight.  LDS holds 16-byte chunks
// XOR-swizzled by row, so the transpose reads of W (4 consecutive rows) and
// the A-operand reads of x (16 rows, same chunk) spread over the banks.  The
// (BN/16) x MT matrix-core chains (16-column group, 16-row sub-tile) are
// spread over the waves; each runs the segment's 16 K-blocks in order from +0.
static constexpr int SK_BN = 128;
static constexpr int SK_ROWS = 512;   // = KC
static constexpr int SK_QROWS = 128;  // W rows per LDS quarter
static constexpr int SK_WCH = SK_BN / 8;           // 16-B chunks per W row
static constexpr int SK_WLD = SK_ROWS * SK_WCH / 512;  // W loads per lane (16)

__device__ __forceinline__ int sk_phys(int row, int chunk) {  // W: element offset of a 16-B chunk
  return row * SK_BN + ((chunk ^ (row & 7)) << 3);
}
__device__ __forceinline__ int sk_xphys(int row, int chunk) {  // x: rows of 64 chunks
  return row * SK_ROWS + ((chunk ^ (row & 15)) << 3);
}
__device__ __forceinline__ int sk_xqphys(int row, int chunk) {  // x quarter: rows of 16 chunks
  return row * SK_QROWS + ((chunk ^ (row & 15)) << 3);
}

// With 64 rows (MT = 4) the x slab of a whole segment would take 64 KB of
// LDS, leaving room for one workgroup per CU; it is staged a quarter (128
// K) at a time instead, beside the W quarter, so that two fit.
template <int MT>  // 16-row sub-tiles of x: 1, 2 or 4
__global__ __launch_bounds__(512, 4) void gemm_skinny_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, float* __restrict__ part,
    int M, int N, int K) {
  constexpr bool XQ = MT == 4;  // x staged by quarters
  __shared__ __attribute__((aligned(16))) uint16_t wl[SK_QROWS * SK_BN];
  __shared__ __attribute__((aligned(16))) uint16_t xl[16 * MT * (XQ ? SK_QROWS : SK_ROWS)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int arow = lane & 15;
  const int tr_r = (lane & 15) >> 2;
  const int tr_c = lane & 3;
  const int n0 = blockIdx.x * SK_BN;
  const int seg = (int)blockIdx.y;
  const int k0 = seg * SK_ROWS;

  const __amdgpu_buffer_rsrc_t wr = make_rsrc(W, (uint32_t)((size_t)K * N * 2));
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
  const uint32_t row_bytes = (uint32_t)N * 2;

  // x slab: chunk c = tid + 512 i is row c/64, 16-B chunk c%64 of the
  // segment (k past K, within a row, is never multiplied: such K-blocks are
  // skipped below)
  // (XQ: load 2q + h is quarter q, chunk c = tid + 512 h: row c/16, chunk
  // 16 q + c%16 of the segment)
  u32x4_t xreg[2 * MT];
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i) {
    int r, ch;
    if constexpr (XQ) {
      const int c = tid + 512 * (i & 1);
      r = c >> 4;
      ch = 16 * (i >> 1) + (c & 15);
    } else {
      const int c = tid + 512 * i;
      r = c >> 6;
      ch = c & 63;
    }
    xreg[i] = bufld128(xr, r < M ? (uint32_t)(r * K + k0 + ch * 8) * 2 : 0x80000000u);
  }
  // W slab: chunk c = tid + 512 i is row c/16, 16-B chunk c%16; loads
  // 4q .. 4q+3 are quarter q.  Rows past K read as zero.  Each W element is
  // read by exactly one workgroup, so the loads carry the non-temporal hint.
  constexpr int RPL = 512 / SK_WCH;  // rows per load (32)
  constexpr int LPQ = SK_QROWS / RPL;  // loads per quarter (4)
  u32x4_t wreg[SK_WLD];
  {
    uint32_t off = (uint32_t)(k0 + tid / SK_WCH) * row_bytes +
                   (uint32_t)(n0 + (tid % SK_WCH) * 8) * 2;
#pragma unroll
    for (int i = 0; i < SK_WLD; ++i) {
      wreg[i] = bufld128_nt(wr, off);
      off += RPL * row_bytes;
    }
  }
  if constexpr (!XQ) {
#pragma unroll
    for (int i = 0; i < 2 * MT; ++i) {
      const int c = tid + 512 * i;
      *(u32x4_t*)&xl[sk_xphys(c >> 6, c & 63)] = xreg[i];
    }
  }

  // chains: (BN/16) column groups x MT sub-tiles over 8 waves; wave w takes
  // column group w % CG and sub-tiles (w / CG) * SPW ..
  constexpr int CG = SK_BN / 16;                 // 8
  constexpr int SPW = MT * CG / 8;               // sub-tiles per wave: MT
  const int cg = wave % CG;
  const int sub0 = (wave / CG) * SPW;
  const int nkb = min(SK_ROWS, K - k0) / KB;
  const int chunk = 2 * cg + (tr_c >> 1);
  const int sub = (tr_c & 1) * 4;
  f32x4_t a[SPW];
#pragma unroll
  for (int i = 0; i < SPW; ++i) a[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (q > 0) {  // every wave is done reading the previous quarter
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
#pragma unroll
    for (int h = 0; h < LPQ; ++h) {
      const int c = tid + 512 * h;  // row c/16 of the quarter, chunk c%16
      *(u32x4_t*)&wl[sk_phys(c / SK_WCH, c % SK_WCH)] = wreg[LPQ * q + h];
    }
    if constexpr (XQ) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = tid + 512 * h;
        *(u32x4_t*)&xl[sk_xqphys(c >> 4, c & 15)] = xreg[2 * q + h];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kb = 4 * q + j;
      if (kb < nkb) {
        const int r0 = j * KB + 8 * g + tr_r;
        const u32x2_t b0 = lds_read_tr16(&wl[sk_phys(r0, chunk) + sub]);
        const u32x2_t b1 = lds_read_tr16(&wl[sk_phys(r0 + 4, chunk) + sub]);
        const u32x4_t bf = u32x4_t{b0.x, b0.y, b1.x, b1.y};
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
          const u32x4_t af =
              XQ ? *(const u32x4_t*)&xl[sk_xqphys((sub0 + i) * 16 + arow, j * 4 + g)]
                 : *(const u32x4_t*)&xl[sk_xphys((sub0 + i) * 16 + arow, kb * 4 + g)];
          a[i] = mfma16x16x32(af, bf, a[i]);
        }
      }
    }
  }
  // N is a multiple of 64, not always of 128: the last tile's upper half
  // (columns >= N, loaded from the next row or as zeros) is never stored
  const int col = n0 + 16 * cg + arow;
  if (n0 + 16 * cg >= N) return;
#pragma unroll
  for (int i = 0; i < SPW; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = (sub0 + i) * 16 + g * 4 + e;
      if (m < M) part[((size_t)seg * M + m) * N + col] = a[i][e];
    }
}

// Ordered fold of segment sums: y = bf16(((p0 + p1) + p2) + ...), fp32.
// One lane per (row, 4 columns).  The loads of up to 32 segments are issued
// together, before any add (one memory round trip for K <= 16384), then
// added in index order.  grid = (ceil(N/256), M), block = 64.
static constexpr int FOLD_BATCH = 32;
__global__ __launch_bounds__(64) void gemm_fold_kernel(const float* __restrict__ part,
                                                       uint16_t* __restrict__ y, int M, int N,
                                                       int S) {
  const int c4 = blockIdx.x * 64 + threadIdx.x;
  const int m = blockIdx.y;
  if (c4 * 4 >= N) return;
  const f32x4_t* p = (const f32x4_t*)(part + (size_t)m * N) + c4;
  const size_t step = (size_t)M * N / 4;
  f32x4_t acc;
  for (int s0 = 0; s0 < S; s0 += FOLD_BATCH) {
    f32x4_t v[FOLD_BATCH];
#pragma unroll
    for (int u = 0; u < FOLD_BATCH; ++u)
      if (s0 + u < S) v[u] = __builtin_nontemporal_load(p + (size_t)(s0 + u) * step);  // read once
    // segment 0 is taken as it is (the fold starts from the first sum)
    acc = s0 == 0 ? v[0] : acc + v[0];
#pragma unroll
    for (int u = 1; u < FOLD_BATCH; ++u)
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
// a segment is issued with a zero accumulator.  Without FOLD or SLICE, one
// chain runs over all of K.  SLICE: the workgroup covers the spw consecutive
// segments of KC from segment blockIdx.y * spw, each from +0, and writes
// every segment's fp32 sum to part[segment][M][N] as it completes; the loads
// run on through the segment boundaries.  (The fast twin slices with KC the
// whole slice and spw = 1.)
//
// Workgroups are dispatched to the 8 XCDs round robin.  remap 2 gives each
// XCD a band of whole tile columns, walked in groups of 4 tile rows, so that
// the 32 workgroups an XCD runs at once share 4 x panels and 8 W panels in
// its L2; remap 1 gives each XCD a contiguous band of tiles, m fastest.
// remap 3 (tile rows a multiple of 8) keeps those 4 x 8 groups but gives
// XCDs x and x + 4 the same band of tile columns, upper and lower half of
// the tile rows, walked in step: each W line is then wanted by two XCDs at
// about the same time, so one of them finds it in the memory-side cache
// rather than HBM (remap 2 reads a band's W twice, half a launch apart).
// Tile index (m fastest: t = column * tm + row) of workgroup `b`.
__device__ __forceinline__ int tile_of_block(int b, int tm, int tn, int remap) {
  int t = b;
  if (remap == 1) {
    t = (t & 7) * ((tm * tn) >> 3) + (t >> 3);
  } else if (remap == 3) {
    const int ncols = tn >> 2, xcd = t & 7, i = t >> 3, pr = xcd & 3, h = xcd >> 2, th = tm >> 1;
    const int first = (i / (4 * ncols)) * 4, gm = min(4, th - first);
    const int r = i - first * ncols;
    t = (pr * ncols + r / gm) * tm + h * th + first + r % gm;
  } else if (remap == 2) {
    const int ncols = tn >> 3, xcd = t & 7, i = t >> 3;
    const int first = (i / (4 * ncols)) * 4, gm = min(4, tm - first);
    const int r = i - first * ncols;
    t = (xcd * ncols + r / gm) * tm + first + r % gm;
  }
  return t;
}

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
    int M, int N, int K, int KC, int tm, int tn, int remap, float* __restrict__ part, int spw) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[3 * TL_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int tr_r = l16 >> 2, tr_c = lane & 3;

  const int t = tile_of_block(blockIdx.x, tm, tn, remap);
  const int m0 = (t % tm) * TL_BM;
  const int n0 = (t / tm) * TL_BN;

  const i32x4_t xr = make_rsrc_words(x, (uint32_t)((size_t)M * K * 2));
  const i32x4_t wr = make_rsrc_words(W, (uint32_t)((size_t)K * N * 2));
  const int seg0 = SLICE ? (int)blockIdx.y * spw : 0;  // first segment (SLICE)
  const int kbeg = SLICE ? seg0 * KC : 0;
  const int kend = SLICE ? min(K, kbeg + spw * KC) : K;
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
  // SLICE: sixteen partial-sum stores per lane go out at each segment
  // boundary, after the loads of the next two stages.  Stores count in vmcnt
  // and complete in issue order, so the first two stages after a boundary
  // wait for vmcnt(22) (their stage's six loads done; the next stage's six
  // and the sixteen stores may be in flight) instead of vmcnt(6), and the
  // ring keeps running.  The stores are issued unconditionally (out-of-range
  // offsets are dropped by the buffer range check), so the count is exact.
  auto stage = [&](int st, auto zero, bool after_store) {
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
    if (SLICE && after_store)
      asm volatile("s_waitcnt vmcnt(22) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
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
  const int wrow0 = m0 + wm * 64;
  // SLICE: the sixteen stores of segment sg's sums, one per (row group,
  // column group) of the wave, each issued whatever the row and column
  // (offsets of rows >= M or columns >= N lie past the buffer and are
  // dropped).  The buffer starts at the tile's corner in part[sg], so the
  // offsets stay below 256 N 4 bytes.
  auto store_part = [&](int sg) {
    const __amdgpu_buffer_rsrc_t pr =
        make_rsrc(part + ((size_t)sg * M + m0) * N + n0,
                  (uint32_t)min((size_t)0x7fffffff, ((size_t)min(TL_BM, M - m0) * N) * 4));
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int r = wm * 64 + s * 16 + l16;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int c = wn * 64 + tt * 16 + g * 4;
        // bit 31 set: past the buffer (at most 2^31 - 1 bytes).  Written as
        // arithmetic, not a select, so that no branch can skip a store.
        const uint32_t out = (uint32_t)(m0 + r >= M) | (uint32_t)(n0 + c >= N);
        const uint32_t off = ((uint32_t)(r * N + c) * 4u) | (out << 31);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[s][tt]), pr, off, 0, 0);
      }
    }
  };

  const int sps = (FOLD || SLICE) ? KC / TL_BK : nstage;  // stages per segment
  int st = 0, sg = seg0;
  for (;;) {
    const int seg_end = min(nstage, st + sps);
    if constexpr (SLICE) {  // the first two stages of a segment wait past its boundary stores
      stage(st++, std::true_type{}, sg > seg0);
      if (st < seg_end) stage(st++, std::false_type{}, sg > seg0);
    } else {
      stage(st++, std::true_type{}, false);
    }
    for (; st < seg_end; ++st) stage(st, std::false_type{}, false);
    if (st >= nstage) break;
    if (FOLD) fold();
    if (SLICE) store_part(sg);
    ++sg;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (FOLD) fold();
  if (SLICE) {
    store_part(sg);
    return;
  }

#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int m = wrow0 + s * 16 + l16;
    if (m < M && n0 + wn * 64 < N) {  // N is a multiple of 64: a wave's columns are all in or out
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const f32x4_t v = FOLD ? tot[s][tt] : acc[s][tt];
        const int col = n0 + wn * 64 + tt * 16 + g * 4;
        *(u32x2_t*)&y[(size_t)m * N + col] =
            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Ring kernel with one K-block per stage: BM x BN tiles of WGM x WGN waves
// ---------------------------------------------------------------------------
// The same arithmetic as gemm_tile_kernel (one v_mfma_f32_16x16x32_bf16 per
// 32-deep K-block, issued as y^T = W^T x^T; with FOLD, segments of 512 from
// +0 folded left to right in registers) on other tile shapes:
//   128 x 128, FOLD (8 waves of 64 x 32, two workgroups per CU): the
//     invariant schedule where 256 x 128 tiles would leave CUs idle but
//     128 x 128 tiles fill the chip (e.g. o and down at M = 1024), so every
//     segment stays in registers instead of going through the workspace;
//   64 x 128, FOLD (4 waves of 32 x 64): the same where only tiles of 64
//     rows fill the chip (o and down at M = 512);
//   256 x 192, FOLD (8 waves of 64 x 96, one workgroup per CU, 251
//     registers): the invariant schedule where 256 x 128 tiles would leave a
//     partial round and 256 x 192 tiles make whole ones (qkv at M = 2048);
//   256 x 256, one chain over all of K (8 waves of 64 x 128): the fast
//     twin's large-M tile, half the L2 bytes per flop of 256 x 128.  The
//     invariant schedule cannot use it: the fold's running total doubles the
//     accumulator registers, which at 256 x 256 exceed the register file.
// The ring holds NS stages of one K-block each (x slab BM rows x 64 B, W slab
// 32 rows x BN*2 B) filled by direct-to-LDS loads NS - 1 stages ahead, one
// barrier per stage.  One set of fragments: each W fragment of the first
// half of the columns is reloaded with the next stage's once that half has
// issued, each x fragment once its row has, the second half's W fragments at
// the end of the stage.
//
// LDS swizzles (16-byte chunks, XOR of the chunk index with row bits), so
// that every read of a fragment touches each bank once:
//   x: rows of 4 chunks; chunk ^ ((row >> 2) & 3) -- a 16-lane read of one
//      chunk of 16 consecutive rows covers all banks;
//   W: rows of BN/8 chunks; the transpose read of 8 k-rows x 2 chunks per
//      32 lanes needs the 8 rows on distinct chunk slots: chunk ^ wsw(row).
template <int BN>
__device__ __forceinline__ int wide_wsw(int r) {
  if constexpr ((BN * 2) % 256 == 0)  // rows a multiple of 256 B: same bank base
    return ((r & 3) << 1) | (r & 8);
  else  // 384-B rows (BN = 192): odd rows start half-way round the banks
    return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2);
}

// s_waitcnt vmcnt(N) then s_barrier, N a compile-time count.  Written as
// inline assembly: the loads it waits for are issued from inline assembly,
// which the compiler's own counter tracking does not see.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int BM, int BN, int WGM, int WGN, int NS, bool FOLD>
__global__ __launch_bounds__(64 * WGM * WGN, BM * BN <= 128 * 128 ? 2 : 1) void gemm_wide_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, uint16_t* __restrict__ y,
    int M, int N, int K, int tm, int tn, int remap, int n_base) {
  constexpr int NW = WGM * WGN;
  constexpr int TM = BM / WGM, TN = BN / WGN;  // wave tile
  constexpr int SM = TM / 16, SN = TN / 16;    // 16 x 16 sub-tiles per wave
  constexpr int XS = BM * 32;                  // x slab elements per stage
  constexpr int WS = 32 * BN;                  // W slab elements per stage
  constexpr int STAGE = XS + WS;
  constexpr int XL = XS * 2 / 1024, WL = WS * 2 / 1024;  // 1 KB wave loads per stage
  // Either every wave loads XL / NW of the x slab and WL / NW of the W slab
  // (EVEN), or, where those do not divide, the first NW / 2 waves load the x
  // slab and the others the W slab (e.g. 256 x 192 on 8 waves: 4 x loads
  // for each of waves 0-3, 3 W loads for each of waves 4-7).
  constexpr bool EVEN = XL % NW == 0 && WL % NW == 0;
  constexpr int NXW = NW / 2;
  static_assert(EVEN || (XL % NXW == 0 && WL % (NW - NXW) == 0), "loads must split over the waves");
  constexpr int XPW = EVEN ? XL / NW : XL / NXW;         // x loads per (x-loading) wave per stage
  constexpr int WPW = EVEN ? WL / NW : WL / (NW - NXW);  // W loads per (W-loading) wave per stage
  constexpr int LPW = EVEN ? XPW + WPW : (XPW > WPW ? XPW : WPW);  // offsets a wave keeps
  constexpr int WCH = BN / 8;                  // 16-B chunks per W row
  constexpr int SPS = 512 / 32;                // stages per segment (KC = 512)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int g = lane >> 4, l16 = lane & 15;
  const int tr_r = l16 >> 2, tr_c = lane & 3;

  const int t = tile_of_block(blockIdx.x, tm, tn, remap);
  const int m0 = (t % tm) * BM;
  const int n0 = n_base + (t / tm) * BN;  // tiles of columns [n_base, N)
  const i32x4_t xr = make_rsrc_words(x, (uint32_t)((size_t)M * K * 2));
  const i32x4_t wr = make_rsrc_words(W, (uint32_t)((size_t)K * N * 2));
  const int nst = K / 32;

  // this wave's loads: x regions xi + j (16 rows of 64 B each) and W
  // regions wi + j (1 KB of the 32 x BN slab); not EVEN, a wave loads only x
  // (xw) or only W
  const bool xw = EVEN || wave < NXW;  // uniform per wave
  const int xi = wave * XPW;
  const int wi = EVEN ? wave * WPW : (wave - NXW) * WPW;
  auto x_off = [&](int region) {
    const int c = region * 64 + lane, r = c >> 2, lc = (c & 3) ^ ((r >> 2) & 3);
    return ((uint32_t)(m0 + r) * (uint32_t)K + (uint32_t)(lc * 8)) * 2u;
  };
  auto w_off = [&](int region) {
    const int c = region * 64 + lane, r = c / WCH;
    const int lc = (c % WCH) ^ wide_wsw<BN>(r);
    return ((uint32_t)r * (uint32_t)N + (uint32_t)(n0 + lc * 8)) * 2u;
  };
  uint32_t goff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    if constexpr (EVEN)
      goff[j] = j < XPW ? x_off(xi + j) : w_off(wi + j - XPW);
    else
      goff[j] = xw ? x_off(xi + (j < XPW ? j : 0)) : w_off(wi + (j < WPW ? j : 0));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(BI_LDS void*)lds;
  // loads of stage st into ring slot st % NS; the stage's advance along K
  // is the scalar offset, and past the last stage it is 2^31, outside the
  // buffer (zeros, no traffic), so that every stage issues exactly LPW
  // loads per wave and the counter waits hold
  auto dma = [&](int st) {
    const bool valid = st < nst;
    const uint32_t base = lds0 + (uint32_t)((st % NS) * STAGE * 2);
    const uint32_t sx = valid ? (uint32_t)(st * 64) : 0x80000000u;
    const uint32_t sw = valid ? (uint32_t)st * 32u * (uint32_t)N * 2u : 0x80000000u;
    if constexpr (EVEN) {
#pragma unroll
      for (int j = 0; j < LPW; ++j) {
        if (j < XPW)
          lds_dma16_so(xr, goff[j], sx, base + (uint32_t)((xi + j) * 1024));
        else
          lds_dma16_so(wr, goff[j], sw, base + (uint32_t)(XS * 2 + (wi + j - XPW) * 1024));
      }
    } else if (xw) {
#pragma unroll
      for (int j = 0; j < XPW; ++j)
        lds_dma16_so(xr, goff[j], sx, base + (uint32_t)((xi + j) * 1024));
    } else {
#pragma unroll
      for (int j = 0; j < WPW; ++j)
        lds_dma16_so(wr, goff[j], sw, base + (uint32_t)(XS * 2 + (wi + j) * 1024));
    }
  };
  // s_waitcnt vmcnt(loads of n stages) + s_barrier for this wave's count
  auto wait_stages = [&](auto n) {
    constexpr int S = decltype(n)::value;
    if constexpr (EVEN)
      wait_vm_barrier<LPW * S>();
    else if (xw)
      wait_vm_barrier<XPW * S>();
    else
      wait_vm_barrier<WPW * S>();
  };

  // fragment addresses (bytes in LDS) in the ring slot of the stage being
  // read, advanced by one slot per stage
  uint32_t xadr = lds0 + (uint32_t)(((wm * TM + l16) * 32 + ((g ^ ((l16 >> 2) & 3)) << 3)) * 2);
  uint32_t wadr[SN][2];
#pragma unroll
  for (int tt = 0; tt < SN; ++tt) {
    const int col = wn * TN + tt * 16 + 4 * tr_c;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 8 * g + 4 * h + tr_r;
      wadr[tt][h] = lds0 + (uint32_t)((XS + r * BN + (((col >> 3) ^ wide_wsw<BN>(r)) << 3) +
                                       (col & 7)) * 2);
    }
  }
  auto advance = [&](int st) {  // from the slot of stage st to that of st + 1
    const uint32_t d = (st % NS == NS - 1) ? (uint32_t)(-(NS - 1) * STAGE * 2)
                                           : (uint32_t)(STAGE * 2);
    xadr += d;
#pragma unroll
    for (int tt = 0; tt < SN; ++tt) {
      wadr[tt][0] += d;
      wadr[tt][1] += d;
    }
  };
  // One set of fragments, each reloaded with the next stage's as soon as
  // the ops that read it have issued.
  u32x4_t xf[SM], wf[SN];
  auto read_w = [&](int tt) {
    const u32x2_t b0 = lds_read_tr16_at(wadr[tt][0]);
    const u32x2_t b1 = lds_read_tr16_at(wadr[tt][1]);
    wf[tt] = u32x4_t{b0.x, b0.y, b1.x, b1.y};
  };
  auto read_x = [&](int sm) {
    xf[sm] = *(const BI_LDS u32x4_t*)(uintptr_t)(xadr + (uint32_t)(sm * 16 * 32 * 2));
  };

  f32x4_t acc[SM][SN];
  f32x4_t tot[FOLD ? SM : 1][FOLD ? SN : 1];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // -0 + s == s exactly for every s, so the first fold copies the first
  // segment's sum bit for bit
#pragma unroll
  for (int i = 0; i < (FOLD ? SM : 1); ++i)
#pragma unroll
    for (int j = 0; j < (FOLD ? SN : 1); ++j) tot[i][j] = f32x4_t{-0.f, -0.f, -0.f, -0.f};
  // one 4-wide group at a time, so that only four accumulator values are
  // copied out of the accumulator registers at once
  auto fold = [&]() {
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        tot[i][j] = tot[i][j] + acc[i][j];
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // Stage st's K-block from the registers in two halves of the columns.
  // The first half's W fragments are reloaded (stage st + 1) once it has
  // issued, each x fragment once its row of the second half has, and the
  // second half's W fragments at the end; the next stage needs them only
  // after its first half.  A segment's first K-block starts from zero.
  constexpr int SH = SN / 2;
  auto stage = [&](int st, auto zero) {
    constexpr bool Z = decltype(zero)::value;
    // this wave's loads of stage st + 1 have landed (stages st + 2 ..
    // st + NS - 2 may be in flight); after the barrier every wave's have,
    // and every wave has consumed the fragments of stage st - 1, so that
    // slot takes stage st + NS - 1
    wait_stages(std::integral_constant<int, NS - 3>{});
    dma(st + NS - 1);
    advance(st);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sm = 0; sm < SM; ++sm)
#pragma unroll
      for (int tt = 0; tt < SH; ++tt)
        acc[sm][tt] = mfma16x16x32(wf[tt], xf[sm], Z ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[sm][tt]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = 0; tt < SH; ++tt) read_w(tt);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sm = 0; sm < SM; ++sm) {
#pragma unroll
      for (int tt = SH; tt < SN; ++tt)
        acc[sm][tt] = mfma16x16x32(wf[tt], xf[sm], Z ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[sm][tt]);
      __builtin_amdgcn_sched_barrier(0);
      read_x(sm);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int tt = SH; tt < SN; ++tt) read_w(tt);
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: stages 0 .. NS - 2 in flight; stage 0's fragments read
#pragma unroll
  for (int s0 = 0; s0 < NS - 1; ++s0) dma(s0);
  wait_stages(std::integral_constant<int, NS - 2>{});
#pragma unroll
  for (int tt = 0; tt < SN; ++tt) read_w(tt);
#pragma unroll
  for (int sm = 0; sm < SM; ++sm) read_x(sm);
  // Segments of SPS stages (FOLD; else one run over all of K).
  int st = 0;
  for (;;) {
    const int seg_end = FOLD ? min(nst, st + SPS) : nst;
    stage(st, std::true_type{});
    for (++st; st < seg_end; ++st) stage(st, std::false_type{});
    if constexpr (FOLD) fold();
    if (st >= nst) break;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int sm = 0; sm < SM; ++sm) {
    const int m = m0 + wm * TM + sm * 16 + l16;
    if (m < M) {
#pragma unroll
      for (int tt = 0; tt < SN; ++tt) {
        const int col = n0 + wn * TN + tt * 16 + g * 4;
        if (n0 + wn * TN + tt * 16 < N) {  // N is a multiple of 16: sub-tiles all in or out
          const f32x4_t v = FOLD ? tot[sm][tt] : acc[sm][tt];
          *(u32x2_t*)&y[(size_t)m * N + col] =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
      }
    }
  }
}

template __global__ void gemm_wide_kernel<64, 128, 2, 2, 6, true>(const uint16_t*,
                                                                  const uint16_t*, uint16_t*, int,
                                                                  int, int, int, int, int, int);
template __global__ void gemm_wide_kernel<128, 128, 2, 4, 5, true>(const uint16_t*,
                                                                   const uint16_t*, uint16_t*, int,
                                                                   int, int, int, int, int, int);
template __global__ void gemm_wide_kernel<256, 192, 4, 2, 5, true>(const uint16_t*,
                                                                   const uint16_t*, uint16_t*, int,
                                                                   int, int, int, int, int, int);
template __global__ void gemm_wide_kernel<256, 256, 2, 4, 4, false>(const uint16_t*,
                                                                    const uint16_t*, uint16_t*, int,
                                                                    int, int, int, int, int, int);

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
static constexpr int BI_KC = 512;  // invariant segment length
static constexpr int TILE_BM = TL_BM;  // rows per tile-kernel workgroup (8 waves)
static constexpr int SKINNY_MAX_M = 64;

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Which kernels run for (M, N, K).  The bits of bi_gemm never depend on it.
static constexpr int TILE_MIN_TILES = 192;  // fewer tiles than this leave CUs idle

// Invariant schedule, M > 64: 256 x 128 tiles with every segment in registers
// when there are enough of them; else 128 x 128 tiles with every segment in
// registers when those fill the chip (o and down at M = 1024: 256 tiles
// instead of 128, and no segment sums through memory); else 64 x 128 tiles
// the same way when those fill it (o and down at M = 512: 256 tiles, where
// the K-slice path wrote and re-read 28 segment sums per output of down);
// else the K-slice path.  The fast twin has no 128 x 128 or 64 x 128 path at
// M > 64 (it slices K freely instead).  M <= 64: the skinny kernel, or
// 128 x 128 tiles for wide N.
enum class GemmPath { Tile, Fold128, Fold64, TileSlice, Skinny };
static constexpr int FOLD128_MIN_M = 16;  // below it the skinny kernel streams W faster
static GemmPath gemm_path(int64_t M, int64_t N, bool fast) {
  if (M <= SKINNY_MAX_M) {
    // 16-64 rows with enough 128 x 128 tiles to fill the chip (gate_up, an LM
    // head): the register-fold tiles beat the skinny kernel and its fold
    // launch (gate_up at M = 64: 55 against 71 us).  The fast twin follows
    // the same choice at these M, as it does for the skinny kernel.
    if (M >= FOLD128_MIN_M && ceil_div(M, 128) * ceil_div(N, 128) >= TILE_MIN_TILES)
      return GemmPath::Fold128;
    return GemmPath::Skinny;
  }
  if (ceil_div(M, TILE_BM) * ceil_div(N, TL_BN) >= TILE_MIN_TILES) return GemmPath::Tile;
  if (!fast && ceil_div(M, 128) * ceil_div(N, 128) >= TILE_MIN_TILES) return GemmPath::Fold128;
  if (!fast && ceil_div(M, 64) * ceil_div(N, 128) >= TILE_MIN_TILES) return GemmPath::Fold64;
  return GemmPath::TileSlice;
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
// The K-slice kernel addresses a tile's partial sums with 32-bit offsets
// below 2^31 (256 rows of N floats).
static constexpr int64_t SLICE_MAX_N = 1 << 21;

// Segments per workgroup on the invariant K-slice path: the count g whose
// critical path, g segments times the rounds that tiles * ceil(S / g)
// workgroups take on a 256-CU chip, is shortest (the largest such g: fewer
// workgroups, fewer pipeline fills).  Each segment is still summed from +0
// and stored on its own, so g moves work between workgroups and never
// changes the bits.
static int64_t segments_per_slice(int64_t tiles, int64_t S) {
  int64_t best = 1, best_cost = INT64_MAX;
  for (int64_t g = 1; g <= S; ++g) {
    const int64_t cost = g * ceil_div(tiles * ceil_div(S, g), 256);
    if (cost <= best_cost) {
      best = g;
      best_cost = cost;
    }
  }
  return best;
}

static int64_t slice_kc(int64_t M, int64_t N, int64_t K, bool fast, int num_cus) {
  return fast ? fast_split_kc(M, N, K, num_cus) : BI_KC;
}

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, bool fast, int num_cus) {
  const GemmPath p = gemm_path(M, N, fast);
  if (p == GemmPath::Tile || p == GemmPath::Fold128 || p == GemmPath::Fold64) return 0;
  const int64_t kc = p == GemmPath::TileSlice ? slice_kc(M, N, K, fast, num_cus) : BI_KC;
  return (size_t)ceil_div(K, kc) * (size_t)M * (size_t)N * sizeof(float);
}

// Tile order of the tile kernel (see remap in gemm_tile_kernel).
static int tile_remap(int64_t tm, int64_t tn) {
  return (tm % 8 == 0 && tn % 4 == 0) ? 3 : (tn % 8 == 0) ? 2 : ((tm * tn) % 8 == 0) ? 1 : 0;
}

// The invariant schedule on 256 x 128 tiles.  Where those leave a partial
// last round of the CUs but 256 x 192 tiles make whole rounds, the 256 x 192
// register-fold tile runs instead (8 waves of 64 x 96).  Otherwise, when the
// 256 x 128 tiles take more than one round and the last is partial, the tile
// columns of that round are computed as 128 x 128 tiles (twice as many, each
// half the work, one per CU in a second launch): e.g. gate_up at M = 1024,
// 896 tiles, runs 768 of 256 x 128 and then 256 of 128 x 128.  All these
// kernels compute every output with the same schedule, so which one computes
// a column changes no bits.
static int launch_tile_invariant(const uint16_t* x, const uint16_t* W, uint16_t* y, int64_t M,
                                 int64_t N, int64_t K, int64_t tm, int64_t tn, hipStream_t stream) {
  const int64_t C = 256;  // rounds of a 256-CU chip (a constant: the plan reads no device state)
  const int64_t T = tm * tn;
  // 256 x 192 tiles where they make whole rounds and 256 x 128 tiles do not
  // (qkv at M = 2048: 256 tiles, one round, where 256 x 128 makes 384)
  if (T % C != 0 && N % 192 == 0 && (tm * (N / 192)) % C == 0) {
    const int64_t tn3 = N / 192;
    hipLaunchKernelGGL((gemm_wide_kernel<256, 192, 4, 2, 5, true>), dim3((unsigned)(tm * tn3)),
                       dim3(512), 0, stream, x, W, y, (int)M, (int)N, (int)K, (int)tm, (int)tn3,
                       tile_remap(tm, tn3), 0);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
  }
  int64_t k = 0;  // tile columns moved to the 128 x 128 launch
  if (T > C && T % C != 0) {
    k = ceil_div(T % C, tm);
    if (k >= tn || ceil_div(M, 128) * k > C) k = 0;  // the 128 x 128 tiles must fit one round
  }
  const int64_t tn1 = tn - k;
  hipLaunchKernelGGL((gemm_tile_kernel<true, false>), dim3((unsigned)(tm * tn1)), dim3(512), 0,
                     stream, x, W, y, (int)M, (int)N, (int)K, BI_KC, (int)tm, (int)tn1,
                     tile_remap(tm, tn1), (float*)nullptr, 1);
  if (hipGetLastError() != hipSuccess) return BI_ERR_HIP;
  if (k == 0) return BI_OK;
  const int64_t tm2 = ceil_div(M, 128), tn2 = ceil_div(N - tn1 * TL_BN, 128);
  hipLaunchKernelGGL((gemm_wide_kernel<128, 128, 2, 4, 5, true>), dim3((unsigned)(tm2 * tn2)),
                     dim3(512), 0, stream, x, W, y, (int)M, (int)N, (int)K, (int)tm2, (int)tn2,
                     tile_remap(tm2, tn2), (int)(tn1 * TL_BN));
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

// The skinny kernel for M <= 64, x padded to 16, 32 or 64 rows: the S
// segment sums of every 128-column tile into part [S][M][N].
static int launch_skinny(const uint16_t* x, const uint16_t* W, float* part, int64_t M, int64_t N,
                         int64_t K, int64_t S, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(N, SK_BN), (unsigned)S);
  if (M <= 16)
    hipLaunchKernelGGL(gemm_skinny_kernel<1>, grid, dim3(512), 0, stream, x, W, part, (int)M,
                       (int)N, (int)K);
  else if (M <= 32)
    hipLaunchKernelGGL(gemm_skinny_kernel<2>, grid, dim3(512), 0, stream, x, W, part, (int)M,
                       (int)N, (int)K);
  else
    hipLaunchKernelGGL(gemm_skinny_kernel<4>, grid, dim3(512), 0, stream, x, W, part, (int)M,
                       (int)N, (int)K);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

int launch_gemm(const uint16_t* x, const uint16_t* W, uint16_t* y, int64_t M, int64_t N,
                int64_t K, void* ws, size_t ws_bytes, hipStream_t stream, bool fast, int num_cus) {
  const int64_t S = ceil_div(K, BI_KC);
  const GemmPath p = gemm_path(M, N, fast);
  if (p == GemmPath::Fold128) {
    const int64_t tm = ceil_div(M, 128), tn = ceil_div(N, 128);
    hipLaunchKernelGGL((gemm_wide_kernel<128, 128, 2, 4, 5, true>), dim3((unsigned)(tm * tn)),
                       dim3(512), 0, stream, x, W, y, (int)M, (int)N, (int)K, (int)tm, (int)tn,
                       tile_remap(tm, tn), 0);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
  }
  if (p == GemmPath::Fold64) {
    const int64_t tm = ceil_div(M, 64), tn = ceil_div(N, 128);
    hipLaunchKernelGGL((gemm_wide_kernel<64, 128, 2, 2, 6, true>), dim3((unsigned)(tm * tn)),
                       dim3(256), 0, stream, x, W, y, (int)M, (int)N, (int)K, (int)tm, (int)tn,
                       tile_remap(tm, tn), 0);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
  }
  if (p == GemmPath::Tile || p == GemmPath::TileSlice) {
    const int64_t tm = ceil_div(M, TILE_BM), tn = ceil_div(N, TL_BN);
    const int remap = tile_remap(tm, tn);
    if (p == GemmPath::Tile) {
      dim3 grid((unsigned)(tm * tn));
      const int64_t tn2 = ceil_div(N, 256);
      if (fast && tm * tn2 >= TILE_MIN_TILES)  // 256 x 256 tiles still fill the chip
        hipLaunchKernelGGL((gemm_wide_kernel<256, 256, 2, 4, 4, false>), dim3((unsigned)(tm * tn2)),
                           dim3(512), 0, stream, x, W, y, (int)M, (int)N, (int)K, (int)tm,
                           (int)tn2, tile_remap(tm, tn2), 0);
      else if (fast)
        hipLaunchKernelGGL((gemm_tile_kernel<false, false>), grid, dim3(512), 0, stream, x, W, y,
                           (int)M, (int)N, (int)K, (int)K, (int)tm, (int)tn, remap, (float*)nullptr,
                           1);
      else
        return launch_tile_invariant(x, W, y, M, N, K, tm, tn, stream);
      return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
    }
    const int64_t kc = slice_kc(M, N, K, fast, num_cus);
    const int64_t ns = ceil_div(K, kc);
    if (ns > 65535 || N > SLICE_MAX_N) return BI_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < (size_t)ns * (size_t)M * (size_t)N * sizeof(float)) return BI_ERR_WORKSPACE;
    float* part = (float*)ws;
    const int64_t spw = fast ? 1 : segments_per_slice(tm * tn, ns);
    hipLaunchKernelGGL((gemm_tile_kernel<false, true>),
                       dim3((unsigned)(tm * tn), (unsigned)ceil_div(ns, spw)), dim3(512), 0, stream,
                       x, W, y, (int)M, (int)N, (int)K, (int)kc, (int)tm, (int)tn, remap, part,
                       (int)spw);
    if (hipGetLastError() != hipSuccess) return BI_ERR_HIP;
    hipLaunchKernelGGL(gemm_fold_kernel, dim3((unsigned)ceil_div(N, 256), (unsigned)M), dim3(64),
                       0, stream, part, y, (int)M, (int)N, (int)ns);
    return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
  }
  if (S > 65535) return BI_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < (size_t)S * (size_t)M * (size_t)N * sizeof(float)) return BI_ERR_WORKSPACE;
  float* part = (float*)ws;
  if (launch_skinny(x, W, part, M, N, K, S, stream) != BI_OK) return BI_ERR_HIP;
  hipLaunchKernelGGL(gemm_fold_kernel, dim3((unsigned)ceil_div(N, 256), (unsigned)M), dim3(64),
                     0, stream, part, y, (int)M, (int)N, (int)S);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

// Segment sums only ([S][M][N] fp32, segment s over K rows [512 s, 512 s +
// 512) from +0): the local half of a row-parallel (K-sharded) GEMM, whose
// ranks gather every rank's segments in rank order and fold them with
// launch_gemm_fold, reproducing the unsharded bits.
int launch_gemm_segments(const uint16_t* x, const uint16_t* W, float* part, int64_t M, int64_t N,
                         int64_t K, hipStream_t stream) {
  const int64_t S = ceil_div(K, BI_KC);
  if (S > 65535) return BI_ERR_UNSUPPORTED;
  if (M <= SKINNY_MAX_M) return launch_skinny(x, W, part, M, N, K, S, stream);
  if (N > SLICE_MAX_N) return BI_ERR_UNSUPPORTED;
  const int64_t tm = ceil_div(M, TILE_BM), tn = ceil_div(N, TL_BN);
  const int remap = tile_remap(tm, tn);
  const int64_t spw = segments_per_slice(tm * tn, S);
  hipLaunchKernelGGL((gemm_tile_kernel<false, true>),
                     dim3((unsigned)(tm * tn), (unsigned)ceil_div(S, spw)), dim3(512), 0, stream,
                     x, W, (uint16_t*)nullptr, (int)M, (int)N, (int)K, BI_KC, (int)tm, (int)tn,
                     remap, part, (int)spw);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

int launch_gemm_fold(const float* part, uint16_t* y, int64_t M, int64_t N, int64_t S,
                     hipStream_t stream) {
  hipLaunchKernelGGL(gemm_fold_kernel, dim3((unsigned)ceil_div(N, 256), (unsigned)M), dim3(64), 0,
                     stream, part, y, (int)M, (int)N, (int)S);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi
