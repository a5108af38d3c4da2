// bi_attn.hip -- paged GQA decode attention, one query token per request.
//
//   out[b,h,:] = softmax_t(scale * q[b,h,:] . k_t) . v_t,  t < ctx_lens[b],
//   kv head of q head h = h / G, G = num_q_heads / num_kv_heads.
//
// The Vosti abstract asks for outputs that do not move with the batch or the
// paged KV layout; the Determinism article (section 4) fixes every split by
// the data and combines partials in a fixed order.  Schedule of the
// batch-invariant entry point, fixed by nothing but the token positions:
//   chunk c = tokens [256c, 256c + 256) of the request, one workgroup per
//   (chunk, kv head, request); inside it, tiles of 64 tokens in order with an
//   online softmax per q head:
//     s_t   = (sum_d q_d k_td on the matrix cores, 32-dim blocks in order) * scale
//     m'    = max(m, max_t s_t);  alpha = exp(m - m') (0 while m = -inf)
//     l     = l * alpha, then l = l + p_t in token order, p_t = exp(s_t - m')
//     acc_d = acc_d * alpha, then acc_d = fma(p_t, v_td, acc_d) in token order
//   the chunk's (m, l, acc[128]) go to an fp32 workspace;
//   a combine kernel folds the chunks of each (request, head) in chunk order:
//     M* = max_c m_c, w_c = exp(m_c - M*), Lsum = fma(l_c, w_c, Lsum),
//     O_d = fma(acc_cd, w_c, O_d), out_d = bf16(O_d / Lsum).
// Which page a token sits in only changes the address it is read from.
//
// The fast twin runs the same kernels with a chunk length picked per
// request from the number of splits that fills the chip for this batch
// (flash-decoding style), so its bits depend on the batch.
#include "bi_common.h"
#include "bi_internal.h"

namespace bi {

static constexpr int AD = 128;        // head_dim
static constexpr int APS = 16;        // page size
static constexpr int ATILE = 64;      // tokens per tile
static constexpr int ACHUNK = 256;    // tokens per chunk (batch-invariant entry point)
static constexpr int APART = AD + 4;  // floats per partial: m, l, 2 pad, acc[128]
static constexpr int AKLD = AD + 8;   // padded K row in LDS (elements)
static constexpr int ACH = 256;       // longest chunk the fast twin may pick (combine bound)
static constexpr int ACOMB_MAXC = 1024;  // chunks per request the combine handles

// Chunk length for request length L: fixed, or (fast twin) from the split count.
__device__ __forceinline__ int chunk_len(int L, int fixed_chunk, int splits) {
  if (fixed_chunk > 0) return fixed_chunk;
  const int per = (L + splits - 1) / splits;
  return ((per + ATILE - 1) / ATILE) * ATILE;
}

// grid = (max chunks, num_kv_heads, batch), block = 256 (4 waves).
// Wave w owns q heads w and w + 4 of the group (G <= 8): lane = token in the
// score phase, lane = pair of dims (2 lane, 2 lane + 1) in the PV phase.
template <int G>
__global__ __launch_bounds__(256) void attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens,
    float* __restrict__ part, int Hq, int Hkv, int max_blocks, long long num_pages, int max_ctx,
    int nc_stride, int fixed_chunk, int splits, float scale) {
  __shared__ __attribute__((aligned(16))) uint16_t qs[G][AD];
  __shared__ __attribute__((aligned(16))) uint16_t ks[ATILE * AKLD];
  __shared__ __attribute__((aligned(16))) uint16_t vs[ATILE * AD];
  __shared__ __attribute__((aligned(16))) float ps[G][ATILE];
  __shared__ int pgs[ACH / APS];  // page ids of the chunk's tokens

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int L = min((int)ctx_lens[b], max_ctx);
  if (L <= 0) return;
  const int C = chunk_len(L, fixed_chunk, splits);
  const int nc = (L + C - 1) / C;
  if (c >= nc) return;
  const int t_begin = c * C;
  const int t_end = min(L, t_begin + C);
  const int32_t* bt = block_table + (size_t)b * max_blocks;

  // q of this kv head's G query heads (bf16, as stored), and the page of
  // every 16 tokens of the chunk (read once, so that the tile loads below
  // do not wait on block-table reads)
  for (int i = tid; i < G * AD; i += 256)
    qs[i / AD][i % AD] = q[((size_t)b * Hq + hk * G) * AD + i];
  if (tid < (t_end - t_begin + APS - 1) / APS) pgs[tid] = bt[t_begin / APS + tid];
  __syncthreads();

  // K/V tile loader: 64 tokens x 16 chunks of 16 B for each of K and V;
  // chunk ci = tid + 256 i: token ci/16, dims 8*(ci%16)..+7.
  u32x4_t kr[4], vr[4];
  auto load_tile = [&](int t0, int nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + 256 * i;
      const int tt = ci >> 4;
      const int dc = ci & 15;
      kr[i] = u32x4_t{0u, 0u, 0u, 0u};
      vr[i] = u32x4_t{0u, 0u, 0u, 0u};
      if (tt < nt) {
        const int t = t0 + tt;
        const long long page = pgs[(t - t_begin) / APS];
        if (page >= 0 && page < num_pages) {
          const size_t kofs = (((size_t)page * 2 + 0) * Hkv + hk) * (APS * AD) + (t % APS) * AD + dc * 8;
          const size_t vofs = kofs + (size_t)Hkv * APS * AD;
          kr[i] = ldg128_nt(kv + kofs);  // each K/V tile is read once per kv head
          vr[i] = ldg128_nt(kv + vofs);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + 256 * i;
      const int tt = ci >> 4;
      const int dc = ci & 15;
      *(u32x4_t*)&ks[tt * AKLD + dc * 8] = kr[i];
      *(u32x4_t*)&vs[tt * AD + dc * 8] = vr[i];
    }
  };

  constexpr int HPW = (G + 3) / 4;  // heads per wave
  float m[HPW], l[HPW], acc0[HPW], acc1[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
    acc0[j] = 0.0f;
    acc1[j] = 0.0f;
  }

  // q of the group as the B operand of the score products: lane l holds
  // head l%16 (zero past G), dims 32 kb + 8 (l/16) .. +7
  u32x4_t bq[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    bq[kb] = (lane & 15) < G ? *(const u32x4_t*)&qs[lane & 15][kb * 32 + (lane >> 4) * 8]
                             : u32x4_t{0u, 0u, 0u, 0u};

  int nt = min(ATILE, t_end - t_begin);
  load_tile(t_begin, nt);
  for (int t0 = t_begin; t0 < t_end; t0 += ATILE) {
    nt = min(ATILE, t_end - t0);
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    const int t1 = t0 + ATILE;
    if (t1 < t_end) load_tile(t1, min(ATILE, t_end - t1));

    // scores on the matrix cores: wave w takes tokens 16w..16w+15 of the
    // tile for every head of the group, S^T = K Q^T, 32-dim blocks in order
    {
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = ks + (16 * wave + (lane & 15)) * AKLD + (lane >> 4) * 8;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sc = mfma16x16x32(*(const u32x4_t*)(krow + kb * 32), bq[kb], sc);
      if ((lane & 15) < G) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ps[lane & 15][16 * wave + (lane >> 4) * 4 + e] = sc[e] * scale;
      }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int hh = wave + 4 * j;
      if (hh < G) {
        // lane = token
        const float s = lane < nt ? ps[hh][lane] : -INFINITY;
        float mt = s;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
        const float mn = fmaxf(m[j], mt);
        const float alpha = (m[j] == -INFINITY) ? 0.0f : __expf(m[j] - mn);
        ps[hh][lane] = (lane < nt) ? __expf(s - mn) : 0.0f;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // l and acc: every lane walks the tokens in order
        float lj = l[j] * alpha;
        float a0 = acc0[j] * alpha;
        float a1 = acc1[j] * alpha;
        const uint32_t* vcol = (const uint32_t*)vs + lane;  // dims 2 lane, 2 lane + 1
        int i = 0;
        // eight tokens at a time: all LDS reads first, then the in-order chain
        for (; i + 8 <= nt; i += 8) {
          const f32x4_t pa = *(const f32x4_t*)&ps[hh][i];
          const f32x4_t pb = *(const f32x4_t*)&ps[hh][i + 4];
          uint32_t v2[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v2[u] = vcol[(i + u) * (AD / 2)];
          const float pv[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            lj = lj + pv[u];
            a0 = __fmaf_rn(pv[u], bf16_lo(v2[u]), a0);
            a1 = __fmaf_rn(pv[u], bf16_hi(v2[u]), a1);
          }
        }
        for (; i < nt; ++i) {
          const float p = ps[hh][i];
          const uint32_t v2 = vcol[i * (AD / 2)];
          lj = lj + p;
          a0 = __fmaf_rn(p, bf16_lo(v2), a0);
          a1 = __fmaf_rn(p, bf16_hi(v2), a1);
        }
        l[j] = lj;
        acc0[j] = a0;
        acc1[j] = a1;
        m[j] = mn;
      }
    }
  }

  // chunk partial: [b][h][c][m, l, -, -, acc[128]]
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hh = wave + 4 * j;
    if (hh < G) {
      float* pp = part + (((size_t)b * Hq + hk * G + hh) * nc_stride + c) * APART;
      if (lane == 0) {
        pp[0] = m[j];
        pp[1] = l[j];
      }
      pp[4 + 2 * lane] = acc0[j];
      pp[5 + 2 * lane] = acc1[j];
    }
  }
}

// ---------------------------------------------------------------------------
// Multi-query (prefill) chunk kernel: the rows of one request share its KV
// cache, so a workgroup takes QB = 64/G consecutive rows of a request (64
// (row, q head) columns) and walks the chunks their contexts reach, loading
// each K/V tile once for all of them.  Every (row, head) gets exactly the
// decode kernel's computation for each chunk:
// the same score instruction on the same operands (an output element of the
// matrix-core product does not depend on the other columns), the same tile
// maxima (a maximum does not depend on order), exponentials and in-order
// chains over the row's own tokens (t < ctx_lens[row]), and the same partial
// layout for the combine.  So a row's output is bitwise the one the decode
// entry point gives it.
//
// Wave w owns columns 16w .. 16w+15.  Scores and softmax run with lane l
// holding column l % 16 (the matrix-core output layout: 16 of the tile's
// tokens per lane); the P V chains run with lane = pair of dims and all 16
// columns advanced together per token, so V is read from LDS once per token
// for 16 columns.  Tokens that every column of the wave takes run without
// masks; the few past the shortest row (the causal diagonal) run per row.
// Chunks start on tile boundaries (256 = 4 x 64), so the walk is one tile
// loop that restarts the online softmax at each chunk start and writes the
// chunk's partials at its end.  grid = num_kv_heads * requests * row blocks
// (1-D), block = 256; the kv head varies fastest (equal work per XCD, which
// take workgroups round-robin), and the row blocks come last-first, so that
// the longest contexts start first.
template <int G>
__global__ __launch_bounds__(256, 3) void attn_prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ row_start,
    const int32_t* __restrict__ ctx_lens, float* __restrict__ part, uint16_t* __restrict__ out,
    int Hq, int Hkv, int requests, int max_blocks, long long num_pages, int max_ctx,
    int nc_stride, int row_blocks, int rows, int cpw, float scale) {
  constexpr int QB = 64 / G;   // rows per workgroup
  constexpr int RPW = 16 / G;  // rows per wave
  constexpr int PU = 1;        // tokens per step of the P V loop
  __shared__ __attribute__((aligned(16))) uint16_t ks[ATILE * AKLD];
  __shared__ __attribute__((aligned(16))) uint16_t vs[ATILE * AD];
  __shared__ __attribute__((aligned(16))) float pw[4][ATILE][16];  // per wave: [token][column]
  __shared__ int lens[QB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hk = (int)(blockIdx.x % (unsigned)Hkv);
  const int z = (int)(blockIdx.x / (unsigned)Hkv);
  const int r = z % requests;
  const int rb = row_blocks - 1 - z / requests;
  // rows outside [0, rows) are never touched, whatever row_start holds
  const long long rs = min(max(0, (int)row_start[r]), rows);
  const long long re = min(max((int)rs, (int)row_start[r + 1]), rows);
  const long long row0l = rs + (long long)rb * QB;
  if (row0l >= re) return;
  const int row0 = (int)row0l;
  const int nrows = (int)min((long long)QB, re - row0l);
  // the block's longest context: one load per lane, then a wave maximum
  const int my_ctx = lane < nrows ? min((int)ctx_lens[row0 + lane], max_ctx) : 0;
  int lmax = my_ctx;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) lmax = max(lmax, __shfl_xor(lmax, o, 64));
  lmax = __builtin_amdgcn_readfirstlane(lmax);
  if (lmax <= 0) return;
  const int32_t* bt = block_table + (size_t)r * max_blocks;

  if (tid < QB) lens[tid] = my_ctx;

  // this lane's column in the score layout, and its q as the B operand
  const int cl = lane & 15;
  const int col = 16 * wave + cl;
  const bool wave_live = 16 * wave < nrows * G;
  u32x4_t bq[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    bq[kb] = col / G < nrows
                 ? ldg128(q + ((size_t)(row0 + col / G) * Hq + hk * G + col % G) * AD + kb * 32 +
                          (lane >> 4) * 8)
                 : u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();
  const int my_len = lens[col / G];

  // K/V tile loader: chunk ci = tid + 256 i is token 16 i + tid/16 of the
  // tile, so every lane needs the same four page ids (scalar loads)
  u32x4_t kr[4], vr[4];
  auto load_tile = [&](int t0, int nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + 256 * i;
      const int tt = ci >> 4;
      const int dc = ci & 15;
      kr[i] = u32x4_t{0u, 0u, 0u, 0u};
      vr[i] = u32x4_t{0u, 0u, 0u, 0u};
      const long long page = 16 * i < nt ? bt[t0 / APS + i] : -1;
      if (tt < nt) {
        const int t = t0 + tt;
        if (page >= 0 && page < num_pages) {
          const size_t kofs = (((size_t)page * 2 + 0) * Hkv + hk) * (APS * AD) + (t % APS) * AD + dc * 8;
          const size_t vofs = kofs + (size_t)Hkv * APS * AD;
          kr[i] = ldg128(kv + kofs);
          vr[i] = ldg128(kv + vofs);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ci = tid + 256 * i;
      const int tt = ci >> 4;
      const int dc = ci & 15;
      *(u32x4_t*)&ks[tt * AKLD + dc * 8] = kr[i];
      *(u32x4_t*)&vs[tt * AD + dc * 8] = vr[i];
    }
  };

  float m_c = -INFINITY, l_c = 0.0f;  // per column (score layout)
  float a0[16], a1[16];               // per column (dims 2 lane, 2 lane + 1)
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    a0[j] = 0.0f;
    a1[j] = 0.0f;
  }
  const uint32_t* vcol = (const uint32_t*)vs + lane;
  const float* pwv = &pw[wave][0][0];

  // this workgroup's chunks: [cpw * blockIdx.y, cpw * blockIdx.y + cpw)
  const int t_lo = (int)blockIdx.y * cpw * ACHUNK;
  const int t_hi = (int)min((long long)lmax, (long long)t_lo + (long long)cpw * ACHUNK);
  if (t_lo >= lmax) return;
  load_tile(t_lo, min(ATILE, t_hi - t_lo));
  for (int t0 = t_lo; t0 < t_hi; t0 += ATILE) {
    // t_hi is lmax or a chunk boundary: tiles never straddle a chunk
    const int nt = min(ATILE, t_hi - t0);
    __syncthreads();  // previous tile fully consumed
    store_tile();
    __syncthreads();
    const int t1 = t0 + ATILE;
    if (t1 < t_hi) load_tile(t1, min(ATILE, t_hi - t1));
    if (!wave_live) continue;
    if (t0 % ACHUNK == 0) {  // a chunk starts: fresh online-softmax state
      m_c = -INFINITY;
      l_c = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        a0[j] = 0.0f;
        a1[j] = 0.0f;
      }
    }

    // scores S^T = K Q^T for the tile's 64 tokens x the wave's 16 columns
    const int nt_c = min(nt, my_len - t0);  // this column's tokens in the tile
    f32x4_t sc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      sc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = ks + (16 * tt + cl) * AKLD + (lane >> 4) * 8;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        sc[tt] = mfma16x16x32(*(const u32x4_t*)(krow + kb * 32), bq[kb], sc[tt]);
    }
    float s[16];
    float mt = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * tt + (lane >> 4) * 4 + e;
        const float sv = sc[tt][e] * scale;
        s[4 * tt + e] = tok < nt_c ? sv : -INFINITY;
        mt = fmaxf(mt, s[4 * tt + e]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const bool live = nt_c > 0;
    const float mn = fmaxf(m_c, mt);
    const float alpha = (m_c == -INFINITY) ? 0.0f : __expf(m_c - mn);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 16 * tt + (lane >> 4) * 4 + e;
        pw[wave][tok][cl] = tok < nt_c ? __expf(s[4 * tt + e] - mn) : 0.0f;
      }
    if (live) {
      l_c = l_c * alpha;
      m_c = mn;
    }
    // tokens taken by every column of the wave, and by the longest
    int ntc = max(nt_c, 0), nmin = ntc, nmax = ntc;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      nmin = min(nmin, __shfl_xor(nmin, o, 64));
      nmax = max(nmax, __shfl_xor(nmax, o, 64));
    }
    nmin = __builtin_amdgcn_readfirstlane(nmin);
    nmax = __builtin_amdgcn_readfirstlane(nmax);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (__builtin_amdgcn_readlane(ntc, j) > 0) {
        const float aj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), j));
        a0[j] = a0[j] * aj;
        a1[j] = a1[j] * aj;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    // all 16 columns, tokens [0, nmin), in token order
    int i = 0;
    for (; i + PU <= nmin; i += PU) {
      uint32_t v2[PU];
      float pl[PU];
      f32x4_t p[PU][4];
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        v2[u] = vcol[(i + u) * (AD / 2)];
        pl[u] = pwv[(i + u) * 16 + cl];
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) p[u][qd] = *(const f32x4_t*)(pwv + (i + u) * 16 + 4 * qd);
      }
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        l_c = l_c + pl[u];
        const float lo = bf16_lo(v2[u]), hi = bf16_hi(v2[u]);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          a0[j] = __fmaf_rn(p[u][j >> 2][j & 3], lo, a0[j]);
          a1[j] = __fmaf_rn(p[u][j >> 2][j & 3], hi, a1[j]);
        }
      }
    }
    for (; i < nmin; ++i) {
      const uint32_t v2 = vcol[i * (AD / 2)];
      l_c = l_c + pwv[i * 16 + cl];
      const float lo = bf16_lo(v2), hi = bf16_hi(v2);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pj = pwv[i * 16 + j];
        a0[j] = __fmaf_rn(pj, lo, a0[j]);
        a1[j] = __fmaf_rn(pj, hi, a1[j]);
      }
    }
    // the rest of each column's tokens [nmin, nt_c), in order
    for (int k = nmin; k < nmax; ++k) {
      const float pk = pwv[k * 16 + cl];
      if (k < nt_c) l_c = l_c + pk;
    }
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      const int nt_r = __builtin_amdgcn_readlane(ntc, rr * G);  // same for the row's G heads
      for (int k = nmin; k < nt_r; ++k) {
        const uint32_t v2 = vcol[k * (AD / 2)];
        const float lo = bf16_lo(v2), hi = bf16_hi(v2);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float pj = pwv[k * 16 + rr * G + h];
          a0[rr * G + h] = __fmaf_rn(pj, lo, a0[rr * G + h]);
          a1[rr * G + h] = __fmaf_rn(pj, hi, a1[rr * G + h]);
        }
      }
    }

    // the chunk ends: partials of the rows whose context reaches it,
    // [row][h][chunk][m, l, -, -, acc].  Column j of the wave is row
    // 16w/G + j/G, head j%G; the strides pass through an empty asm so that
    // the sixteen addresses are formed here rather than held across the loop.
    if (t1 % ACHUNK == 0 || t1 >= t_hi) {
      const int c = t0 / ACHUNK;
      int hs = nc_stride * APART;
      asm volatile("" : "+s"(hs));
      float* pbase = part + ((size_t)(row0 + 16 * wave / G) * Hq + hk * G) * hs + (size_t)c * APART;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (__builtin_amdgcn_readlane(my_len, j) > c * ACHUNK) {
          float* pp = pbase + (size_t)((j / G) * Hq + j % G) * hs;
          if (lane == j) {
            pp[0] = m_c;
            pp[1] = l_c;
          }
          pp[4 + 2 * lane] = a0[j];
          pp[5 + 2 * lane] = a1[j];
        }
      }
    }
  }

  // The combine, as the combine kernel does it, for the wave's columns: the
  // workgroup has written every chunk partial of its rows.  M* = max m_c,
  // w_c = exp(m_c - M*), L and O folded in chunk order, out = bf16(O / L).
  // With the chunks split over workgroups (gridDim.y > 1) the combine kernel
  // runs afterwards instead.
  if (!wave_live || gridDim.y > 1) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  int hs = nc_stride * APART;
  asm volatile("" : "+s"(hs));
  const float* pbase = part + ((size_t)(row0 + 16 * wave / G) * Hq + hk * G) * hs;
  uint16_t* obase = out + ((size_t)(row0 + 16 * wave / G) * Hq + hk * G) * AD + 2 * lane;
  for (int j = 0; j < 16; ++j) {
    if (16 * wave + j >= nrows * G) break;
    const int L = __builtin_amdgcn_readlane(my_len, j);
    uint32_t* o = (uint32_t*)(obase + (size_t)((j / G) * Hq + j % G) * AD);
    if (L <= 0) {
      *o = 0u;
      continue;
    }
    const int nc = min((L + ACHUNK - 1) / ACHUNK, ACOMB_MAXC);
    const float* pp = pbase + (size_t)((j / G) * Hq + j % G) * hs;
    float mx = -INFINITY;
    for (int cc = lane; cc < nc; cc += 64) mx = fmaxf(mx, pp[(size_t)cc * APART]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float ls = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += 8) {
      float mv[8], lv[8], v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* pc = pp + (size_t)min(c0 + u, nc - 1) * APART;
        mv[u] = pc[0];
        lv[u] = pc[1];
        v0[u] = pc[4 + 2 * lane];
        v1[u] = pc[5 + 2 * lane];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < nc) {
          const float w = __expf(mv[u] - mx);
          ls = __fmaf_rn(lv[u], w, ls);
          o0 = __fmaf_rn(v0[u], w, o0);
          o1 = __fmaf_rn(v1[u], w, o1);
        }
      }
    }
    *o = (uint32_t)f32_to_bf16_bits(o0 / ls) | ((uint32_t)f32_to_bf16_bits(o1 / ls) << 16);
  }
}
// grid = (num_q_heads, batch), block = 128 (one lane per dim).
// The chunk maxima and weights are computed by all lanes in parallel (the
// maximum does not depend on order); the two sums then run in chunk order,
// with the partials of 32 chunks fetched before each stretch of the chain.

__global__ __launch_bounds__(128) void attn_combine_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ ctx_lens,
    uint16_t* __restrict__ out, int Hq, int max_ctx, int nc_stride, int fixed_chunk, int splits) {
  __shared__ float wsh[ACOMB_MAXC];
  __shared__ float lsh[ACOMB_MAXC];
  __shared__ float red[2];
  const int d = threadIdx.x;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  uint16_t* o = out + ((size_t)b * Hq + h) * AD;
  const int L = min((int)ctx_lens[b], max_ctx);
  if (L <= 0) {
    o[d] = 0;
    return;
  }
  const int C = chunk_len(L, fixed_chunk, splits);
  const int nc = min((L + C - 1) / C, ACOMB_MAXC);
  const float* pp = part + ((size_t)b * Hq + h) * nc_stride * APART;
  // M* = max_c m_c
  float mx = -INFINITY;
  for (int cc = d; cc < nc; cc += 128) {
    const float mc = pp[(size_t)cc * APART];
    wsh[cc] = mc;
    lsh[cc] = pp[(size_t)cc * APART + 1];
    mx = fmaxf(mx, mc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((d & 63) == 0) red[d >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  // w_c = exp(m_c - M*)
  for (int cc = d; cc < nc; cc += 128) wsh[cc] = __expf(wsh[cc] - mx);
  __syncthreads();
  // Lsum and O_d in chunk order
  float ls = 0.0f, acc = 0.0f;
  const float* pd = pp + 4 + d;
  int cc = 0;
  for (; cc + 32 <= nc; cc += 32) {
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = pd[(size_t)(cc + u) * APART];
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      ls = __fmaf_rn(lsh[cc + u], wsh[cc + u], ls);
      acc = __fmaf_rn(v[u], wsh[cc + u], acc);
    }
  }
  if (cc < nc) {
    // the last stretch: its loads issued together as well (zeros past nc)
    float v[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = cc + u < nc ? pd[(size_t)(cc + u) * APART] : 0.0f;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      if (cc + u < nc) {
        ls = __fmaf_rn(lsh[cc + u], wsh[cc + u], ls);
        acc = __fmaf_rn(v[u], wsh[cc + u], acc);
      }
    }
  }
  o[d] = (uint16_t)f32_to_bf16_bits(acc / ls);  // IEEE division
}

// Split count of the fast twin: enough (request, kv head, split) units for
// four per CU, but never a chunk longer than the kernel's LDS holds.
static int attn_splits(const bi_attn_desc* d, int num_cus) {
  const long long units = (long long)d->batch * d->num_kv_heads;
  long long s = (4LL * num_cus + units - 1) / units;
  const long long maxs = (d->max_ctx_len + ATILE - 1) / ATILE;
  const long long mins = (d->max_ctx_len + ACH - 1) / ACH;
  s = std::max(mins, std::min(s, maxs));
  return (int)std::max(1LL, std::min(s, (long long)ACOMB_MAXC));
}

static int nc_stride_of(const bi_attn_desc* d, bool fast, int num_cus) {
  return fast ? attn_splits(d, num_cus) : (d->max_ctx_len + ACHUNK - 1) / ACHUNK;
}

size_t attn_ws_bytes(const bi_attn_desc* d, bool fast, int num_cus) {
  const size_t nc = (size_t)nc_stride_of(d, fast, num_cus);
  return (size_t)d->batch * d->num_q_heads * nc * APART * sizeof(float);
}

int launch_attn(const uint16_t* q, const uint16_t* kv, const int32_t* block_table,
                const int32_t* ctx_lens, uint16_t* out, const bi_attn_desc* d, void* ws,
                size_t ws_bytes, hipStream_t stream, bool fast, int num_cus) {
  const int G = d->num_q_heads / d->num_kv_heads;
  const int ncs = nc_stride_of(d, fast, num_cus);
  if (ws_bytes < attn_ws_bytes(d, fast, num_cus)) return BI_ERR_WORKSPACE;
  if (ncs > 65535 || d->num_kv_heads > 65535 || d->batch > 65535) return BI_ERR_UNSUPPORTED;
  float* part = (float*)ws;
  const int fixed = fast ? 0 : ACHUNK;
  const int splits = fast ? ncs : 0;
  dim3 grid((unsigned)ncs, (unsigned)d->num_kv_heads, (unsigned)d->batch);
#define BI_ATTN_LAUNCH(GG)                                                                    \
  hipLaunchKernelGGL(attn_chunk_kernel<GG>, grid, dim3(256), 0, stream, q, kv, block_table,  \
                     ctx_lens, part, d->num_q_heads, d->num_kv_heads, d->max_blocks_per_seq, \
                     (long long)d->num_pages, d->max_ctx_len, ncs, fixed, splits, d->scale)
  switch (G) {
    case 1: BI_ATTN_LAUNCH(1); break;
    case 2: BI_ATTN_LAUNCH(2); break;
    case 4: BI_ATTN_LAUNCH(4); break;
    case 8: BI_ATTN_LAUNCH(8); break;
    default: return BI_ERR_UNSUPPORTED;
  }
#undef BI_ATTN_LAUNCH
  if (hipGetLastError() != hipSuccess) return BI_ERR_HIP;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)d->num_q_heads, (unsigned)d->batch),
                     dim3(128), 0, stream, part, ctx_lens, out, d->num_q_heads, d->max_ctx_len,
                     ncs, fixed, splits);
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

int launch_prefill_attn(const uint16_t* q, const uint16_t* kv, const int32_t* block_table,
                        const int32_t* row_start, const int32_t* ctx_lens, uint16_t* out,
                        const bi_attn_desc* d, int requests, int max_rows_per_request, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  const int G = d->num_q_heads / d->num_kv_heads;
  const int ncs = nc_stride_of(d, false, 0);
  if (ws_bytes < attn_ws_bytes(d, false, 0)) return BI_ERR_WORKSPACE;
  const int qb = 64 / G;
  const long long row_blocks = (max_rows_per_request + qb - 1) / qb;
  const long long nwg = (long long)d->num_kv_heads * requests * row_blocks;
  if (nwg > 0x7fffffffLL) return BI_ERR_UNSUPPORTED;
  // Few row blocks (under 2048 workgroups: a verify window of a few rows per
  // request over long contexts): split each block's chunks over several
  // workgroups, toward 8192 in all, and combine in a second kernel.  Many
  // row blocks (a prefill): one workgroup walks all of a block's chunks and
  // combines them itself.  Either way every chunk is computed as in the
  // decode entry point and combined in chunk order, so the split never
  // changes the bits.
  // (the combine kernel's grid has one row of workgroups per query row, at
  // most 65535)
  const long long groups = (nwg >= 2048 || d->batch > 65535)
                               ? 1
                               : std::max(1LL, std::min((long long)ncs, (8192 + nwg - 1) / nwg));
  const int cpw = (int)((ncs + groups - 1) / groups);
  const long long ngy = (ncs + cpw - 1) / cpw;
  if (ngy > 65535) return BI_ERR_UNSUPPORTED;
  float* part = (float*)ws;
#define BI_PREFILL_LAUNCH(GG)                                                                  \
  hipLaunchKernelGGL(attn_prefill_kernel<GG>, dim3((unsigned)nwg, (unsigned)ngy), dim3(256), 0, \
                     stream, q, kv, block_table, row_start, ctx_lens, part, out, d->num_q_heads, \
                     d->num_kv_heads, requests, d->max_blocks_per_seq, (long long)d->num_pages, \
                     d->max_ctx_len, ncs, (int)row_blocks, d->batch, cpw, d->scale)
  switch (G) {
    case 1: BI_PREFILL_LAUNCH(1); break;
    case 2: BI_PREFILL_LAUNCH(2); break;
    case 4: BI_PREFILL_LAUNCH(4); break;
    case 8: BI_PREFILL_LAUNCH(8); break;
    default: return BI_ERR_UNSUPPORTED;
  }
#undef BI_PREFILL_LAUNCH
  if (hipGetLastError() != hipSuccess) return BI_ERR_HIP;
  if (ngy > 1) {
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)d->num_q_heads, (unsigned)d->batch),
                       dim3(128), 0, stream, part, ctx_lens, out, d->num_q_heads, d->max_ctx_len,
                       ncs, ACHUNK, 0);
  }
  return hipGetLastError() == hipSuccess ? BI_OK : BI_ERR_HIP;
}

}  // namespace bi
