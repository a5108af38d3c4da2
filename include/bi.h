/*
 * bi.h -- C ABI of the batch-invariant forward kernels for MI355X (gfx950).
 *
 * Three operations of a Llama-style decoder layer's forward pass -- a bf16
 * GEMM, RMSNorm and paged decode attention -- each written so that every
 * output row's floating-point reduction order is a function of that row's own
 * data only: never of the batch size M, of the other requests in the batch,
 * of where their KV pages sit, of the longest context, or of how many compute
 * units are free.  Each has a "_fast" twin with the same signature that picks
 * its schedule from the batch shape and the CU count (deterministic from run
 * to run, but not batch-invariant); the twins exist to measure the cost of
 * invariance.
 *
 * Sources (web pages, cited by title and section):
 *   [Article] "LLM inference determinism engineering in depth: from float
 *             non-associativity and batch invariance to reproducible kernels"
 *             (ybb.press, ai-applications/14528).
 *   [LLM-42]  "LLM-42: Enabling Determinism in LLM Inference with Verified
 *             Speculation (SOSP 2026)", ai-infra-wiki digest.
 *   [Vosti]   arxivdaily 2609.38981, abstract of the Vosti engine.
 *
 * Conventions for every call:
 *   - Pointers named x, W, y, g, q, kv_pages, block_table, ctx_lens, out and
 *     ws are DEVICE pointers, owned by the caller, 16-byte aligned.  The
 *     library allocates and frees nothing inside a call.
 *   - bf16 values are passed as raw bits (bi_bf16).  Matrices are row-major
 *     and contiguous.
 *   - stream is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work and return; a device-side fault surfaces at the caller's next
 *     synchronisation.
 *   - Errors are reported by the return code only; nothing is printed and
 *     nothing aborts.  On an error nothing is enqueued.
 *   - Workspace: operations that need one take (ws, ws_bytes), sized by the
 *     matching *_workspace_bytes query (0 means ws may be NULL).  It is
 *     scratch: its contents need no initialisation and are undefined after
 *     the call.  One workspace may be reused by any sequence of calls on one
 *     stream; concurrent calls must use distinct workspaces.  A call captured
 *     into a HIP graph keeps its pointers, the workspace's included, for
 *     every replay: the workspace must stay allocated while the graph may be
 *     replayed, and work that uses it between replays must be ordered with
 *     them on the same stream.
 *   - Reentrancy: concurrent calls on different streams with distinct
 *     workspaces are safe.  The library keeps no state that affects a
 *     result; it fills two read-only caches on first use, thread-safely: the
 *     version string and each device's CU count (read only by the _fast
 *     twins).
 *   - Determinism contract (bi_* entry points, not the _fast twins): the
 *     output bits of a row/request depend only on that row's/request's
 *     inputs, the weights, gain or logical KV contents, the library version
 *     and the gfx target.  ([Article] section 4: the reduction order must
 *     depend on the data only; [Vosti]: kernel choice independent of engine
 *     state, cached KV bound to its logical token position.)
 *   - What the plan reads.  The reduction schedule -- which values are
 *     added, in which order, by which instruction -- is fixed by (N, K), by
 *     H, or by (D, page size, Hq, Hkv).  How that schedule's fixed pieces
 *     (16-row matrix-core sub-tiles, 512-row K segments, 256-token chunks)
 *     are grouped into workgroups and kernels reads the batch as well: M
 *     picks the skinny kernel's 16/32/64-row tiles or 64-, 128- or
 *     256-row register-fold tiles (256-row tiles whose last round on 256
 *     compute units would be partial hand that round's columns to 128-row
 *     tiles in a second launch) and, where few tiles would leave compute
 *     units idle, how many consecutive segments one workgroup runs.  That
 *     grouping moves work between workgroups and never changes an output
 *     bit; the GPU tests check every M from 1 to 2048 against the
 *     M = 2048 rows bit for bit.  This is the
 *     reading taken of the Article's fixed-tile rule (section 4): what
 *     must not follow M is the arithmetic each output sees, not the
 *     launch shape.
 */
#ifndef BI_H
#define BI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t bi_bf16;

enum {
    BI_OK = 0,
    BI_ERR_NULL = -1,        /* a required pointer is NULL                   */
    BI_ERR_SHAPE = -2,       /* a size is <= 0 or a size product overflows   */
    BI_ERR_UNSUPPORTED = -3, /* shape outside what the kernels handle, or a
                                pointer not 16-byte aligned                   */
    BI_ERR_WORKSPACE = -4,   /* ws is NULL or ws_bytes smaller than needed   */
    BI_ERR_HIP = -5,         /* the HIP launch itself failed                 */
    BI_ERR_SCRATCH = -6      /* the call needs more scratch than the
                                library's static array holds (bi_gemm_noalloc) */
};

/* Library version, gfx target and every schedule constant, as one static
 * NUL-terminated string.  [Article] section 6: record the exact kernel
 * library and compile flags next to every result. */
const char *bi_version(void);

/* Static text for a status code. */
const char *bi_status_string(int status);

/* ------------------------------------------------------------------------
 * GEMM:  y[M,N] = bf16_rne( x[M,K] . W[K,N] ),  bf16 in, fp32 accumulate.
 *
 * [Article] section 1 (the batch-1 vs batch-8 linear layer), section 2.2
 * (shape-dependent tiling and split-k with float atomics break invariance),
 * section 4 (fixed M tile with padding; K split only into fixed segments whose
 * partial sums go to a fixed workspace and are added in index order; no float
 * atomics), section 5 (no reduced-precision intermediate reduction).
 *
 * Schedule of bi_gemm (fixed by K only): K-blocks of 32 (one
 * v_mfma_f32_16x16x32_bf16), segments of 512 accumulated from +0, segments
 * added left to right 0..S-1 in fp32, S = ceil(K/512), one RNE narrowing.
 *
 * x: [M,K] bf16 row-major.  W: [K,N] bf16 row-major (y = x times W, as the
 * article's section-1 demo multiplies).  y: [M,N] bf16 row-major, written
 * only for rows < M.  Requirements: M, N, K >= 1; K % 32 == 0; N % 64 == 0;
 * M*K, K*N, M*N < 2^31; else BI_ERR_SHAPE / BI_ERR_UNSUPPORTED.
 * ws/ws_bytes: workspace of at least bi_gemm_workspace_bytes(M,N,K) bytes
 * (fp32 segment sums when they have to leave the compute unit; 0 otherwise).
 * ---------------------------------------------------------------------- */
size_t bi_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int bi_gemm(const bi_bf16 *x, const bi_bf16 *W, bi_bf16 *y,
            int64_t M, int64_t N, int64_t K,
            void *ws, size_t ws_bytes, void *stream);

/* Same operation with tiles and K split chosen from (M, N, K) and the CU
 * count.  Deterministic run to run (ordered workspace, no float atomics) but
 * NOT batch-invariant.  Same arguments and requirements. */
size_t bi_gemm_fast_workspace_bytes(int64_t M, int64_t N, int64_t K);
int bi_gemm_fast(const bi_bf16 *x, const bi_bf16 *W, bi_bf16 *y,
                 int64_t M, int64_t N, int64_t K,
                 void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * bi_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments (less the workspace), requirements, schedule
 * and bits as bi_gemm.  The segment sums that bi_gemm sends through a
 * workspace go to a static device array of BI_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends; the
 * call allocates nothing.  A call whose bi_gemm_workspace_bytes(M, N, K)
 * exceeds that size returns BI_ERR_SCRATCH and enqueues nothing (with the
 * Llama-3-8B linears it fits every M <= 64, and M up to about 256 on the
 * 4096-row ones).  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU, on any streams, race on it and must be ordered by
 * the caller.  The array needs no initialisation and keeps the last call's
 * contents.  Its device address is taken on a device's first call, under
 * a lock.
 * ---------------------------------------------------------------------- */
#define BI_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int bi_gemm_noalloc(const bi_bf16 *x, const bi_bf16 *W, bi_bf16 *y,
                    int64_t M, int64_t N, int64_t K, void *stream);

/* ------------------------------------------------------------------------
 * The two halves of bi_gemm's schedule, for a row-parallel (K-sharded)
 * GEMM across ranks: the Article's section 4 design of fixed segments whose
 * sums are combined in a fixed second stage, with the second stage placed
 * after the exchange.  Each rank computes its shard's segment sums; the
 * ranks gather every rank's segments in rank order (an all-gather, whose
 * result does not depend on message size or rank count, unlike a ring or
 * tree all-reduce); each then folds all of them.  When every shard but the
 * last is a multiple of 512 rows of K, the folded y is bitwise bi_gemm's
 * on the unsharded x and W, for any number of ranks.
 *
 * bi_gemm_segments: part[s][m][n] (fp32, [ceil(K/512)][M][N], caller
 *   owned, 16-byte aligned) = sum over k in [512 s, min(512 s + 512, K)) of
 *   x[m][k] W[k][n], accumulated from +0 in bi_gemm's order.  x, W as for
 *   bi_gemm (same requirements, and N <= 2^21 when M > 64, else
 *   BI_ERR_UNSUPPORTED); no workspace.
 * bi_gemm_fold: y[m][n] = bf16(((part[0] + part[1]) + ...) + part[S-1]),
 *   fp32 adds in index order, round to nearest even; part as above with S
 *   segments, M <= 65535, N % 64 == 0, 16-byte aligned pointers.
 * ---------------------------------------------------------------------- */
int bi_gemm_segments(const bi_bf16 *x, const bi_bf16 *W, float *part,
                     int64_t M, int64_t N, int64_t K, void *stream);
int bi_gemm_fold(const float *part, bi_bf16 *y, int64_t M, int64_t N,
                 int64_t S, void *stream);

/* ------------------------------------------------------------------------
 * RMSNorm:  y[m,h] = bf16_rne( (x[m,h] * r_m) * g[h] ),
 *           r_m = 1 / sqrt( (sum_h x[m,h]^2) / H + eps ),  fp32 throughout.
 *
 * [LLM-42] problem statement and [Article] section 2.2: normalization is one
 * of the reductions whose schedule a dynamic batch changes.  bi_rmsnorm
 * reduces each row in one workgroup of 256 lanes with a fixed tree (per-lane
 * strided sums, a 64-lane xor butterfly, four wave sums added in order);
 * sqrt and the division are correctly rounded.
 *
 * x: [M,H] bf16.  g: [H] bf16.  y: [M,H] bf16 (may not alias x).
 * Requirements: M, H >= 1; H % 8 == 0; M*H < 2^31.  No workspace.
 * ---------------------------------------------------------------------- */
int bi_rmsnorm(const bi_bf16 *x, const bi_bf16 *g, bi_bf16 *y,
               int64_t M, int64_t H, float eps, void *stream);

/* Rows per workgroup and lanes per row chosen from M; not batch-invariant. */
int bi_rmsnorm_fast(const bi_bf16 *x, const bi_bf16 *g, bi_bf16 *y,
                    int64_t M, int64_t H, float eps, void *stream);

/* Residual add followed by RMSNorm, the pair that closes each half of a
 * decoder layer, in one pass:
 *   sum[m,h] = bf16_rne(a[m,h] + b[m,h])          (as bi_add)
 *   y = bi_rmsnorm(sum, g, eps)                    (the same tree and bits)
 * a, b, sum, y: [M,H] bf16; sum may be a or b (in-place residual), y must not
 * alias a, b or sum.  g: [H] bf16.  Requirements as bi_rmsnorm, and
 * H <= 8192; else BI_ERR_UNSUPPORTED.  No workspace. */
int bi_add_rmsnorm(const bi_bf16 *a, const bi_bf16 *b, const bi_bf16 *g,
                   bi_bf16 *sum, bi_bf16 *y, int64_t M, int64_t H, float eps,
                   void *stream);

/* ------------------------------------------------------------------------
 * Paged decode attention (one query token per request, GQA):
 *   out[b,h,:] = softmax_t( scale * q[b,h,:] . k_t ) . v_t,  t < ctx_lens[b],
 *   kv head of q head h = h / (num_q_heads / num_kv_heads).
 *
 * [Vosti] abstract: outputs must not change with the batch or with the paged
 * KV-cache layout.  [Article] section 4: split work only at boundaries fixed
 * by the data and combine partials in a fixed order.  bi_paged_decode_attn
 * cuts every request's context into chunks of 256 tokens (tiles of 64 inside
 * a chunk, online softmax), whatever the batch, and combines the chunk
 * partials in chunk order.
 *
 * q:           [batch, num_q_heads, head_dim] bf16.
 * kv_pages:    [num_pages, 2 (K then V), num_kv_heads, page_size, head_dim]
 *              bf16; one (page, K|V, kv head) block is contiguous.
 * block_table: [batch, max_blocks_per_seq] int32; token t of request b sits
 *              in page block_table[b][t / page_size], slot t % page_size.
 *              Entries past a request's last page are never read.
 * ctx_lens:    [batch] int32, read on the device; a request with
 *              ctx_lens[b] <= 0 gets zeros.  Every ctx_lens[b] must be
 *              <= max_ctx_len and every referenced page < num_pages (device
 *              data is not range-checked).
 * out:         [batch, num_q_heads, head_dim] bf16.
 * Supported: head_dim == 128, page_size == 16, num_q_heads / num_kv_heads
 * in {1, 2, 4, 8}, batch >= 1, 1 <= max_ctx_len <= max_blocks_per_seq *
 * page_size and max_ctx_len <= 262144.  max_ctx_len only sizes the grid and
 * the workspace; it never changes the bits.
 * ---------------------------------------------------------------------- */
typedef struct {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_blocks_per_seq;
    int64_t num_pages;
    int32_t max_ctx_len;
    float scale; /* > 0: used as given; <= 0 (or -0): the default
                    1/sqrt(head_dim), computed by the library as the fp32
                    division 1.0f / sqrtf(head_dim); NaN: BI_ERR_UNSUPPORTED */
} bi_attn_desc;

size_t bi_attn_workspace_bytes(const bi_attn_desc *d);
int bi_paged_decode_attn(const bi_bf16 *q, const bi_bf16 *kv_pages,
                         const int32_t *block_table, const int32_t *ctx_lens,
                         bi_bf16 *out, const bi_attn_desc *d,
                         void *ws, size_t ws_bytes, void *stream);

/* Number of KV splits chosen from batch * num_kv_heads against the CU count
 * (split boundaries then depend on the batch): not batch-invariant. */
size_t bi_attn_fast_workspace_bytes(const bi_attn_desc *d);
int bi_paged_decode_attn_fast(const bi_bf16 *q, const bi_bf16 *kv_pages,
                              const int32_t *block_table,
                              const int32_t *ctx_lens, bi_bf16 *out,
                              const bi_attn_desc *d, void *ws, size_t ws_bytes,
                              void *stream);

/* ------------------------------------------------------------------------
 * Multi-query (prefill) attention: many rows of the same requests at once,
 * each with exactly the decode entry point's per-row schedule, so a row's
 * output is bitwise what bi_paged_decode_attn gives it (prefill/decode
 * invariance, the property the LLM-42 digest notes its own method lacks).
 * Rows of a request share its KV cache; a workgroup loads every K/V tile
 * once for up to 64/G rows.  With few rows the chunks of a row block are
 * also split over workgroups and folded in chunk order by the combine of
 * the decode entry point (same bits).
 *
 * q:           [rows, num_q_heads, head_dim] bf16, rows grouped by request.
 * kv_pages:    as for bi_paged_decode_attn.
 * block_table: [requests, max_blocks_per_seq] int32 (one row per REQUEST).
 * row_start:   [requests + 1] int32 (device): the rows of request r are
 *              [row_start[r], row_start[r+1]); row_start[0] = 0,
 *              row_start[requests] = rows, non-decreasing.
 * ctx_lens:    [rows] int32 (device): row m attends to tokens
 *              [0, ctx_lens[m]) of its request (position + 1 for causal
 *              prefill); <= 0 gives zeros.
 * out:         [rows, num_q_heads, head_dim] bf16.
 * d:           as for bi_paged_decode_attn with d->batch = rows.
 * requests:    number of requests R; max_rows_per_request: an upper bound on
 *              row_start[r+1] - row_start[r] (sizes the grid).
 * ws:          at least bi_attn_workspace_bytes(d) bytes.
 * Same requirements as bi_paged_decode_attn, and requests *
 * ceil(max_rows_per_request / (64 / G)) <= 65535.
 * ---------------------------------------------------------------------- */
int bi_paged_prefill_attn(const bi_bf16 *q, const bi_bf16 *kv_pages,
                          const int32_t *block_table, const int32_t *row_start,
                          const int32_t *ctx_lens, bi_bf16 *out,
                          const bi_attn_desc *d, int32_t requests,
                          int32_t max_rows_per_request, void *ws,
                          size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Per-request sampling (the Determinism article, section 6, item 3: a
 * counter-based generator of the Philox family keyed by request and step
 * instead of a shared random stream).  Row m's token depends only on its
 * logits row, seeds[m] and steps[m]:
 *   Philox4x64-10 (Salmon et al., SC 2011) with key (seeds[m], 0) and
 *   counter (v / 4, steps[m], 0, 0); vocabulary entry v takes word v % 4;
 *   u = ((word >> 41) + 1/2) * 2^-23 (fp32, in (0, 1));
 *   temperature[m] > 0: Gumbel-max, score = l / T + (-log(-log u)) in fp32;
 *   temperature[m] <= 0 or NaN: greedy, score = l;
 *   tokens[m] = the first index of the largest score (NaN counts as -inf).
 * logits [M, V] bf16; seeds, steps [M] uint64; temperature [M] fp32;
 * tokens [M] int32 out; all device memory.  1 <= M <= 65535, V < 2^31.
 * ws: scratch of at least bi_sample_workspace_bytes(M) bytes (4-byte
 * aligned, no initialisation): each row's vocabulary is split over 32
 * workgroups whose best (score, index) pairs are then compared; the token
 * does not depend on the split.
 * ---------------------------------------------------------------------- */
size_t bi_sample_workspace_bytes(int64_t M);
int bi_sample(const bi_bf16 *logits, int64_t M, int64_t V,
              const uint64_t *seeds, const uint64_t *steps,
              const float *temperature, int32_t *tokens, void *ws,
              size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Commit or rollback after a grouped verification pass (the LLM-42 digest,
 * method: the prefix the fixed-shape recompute confirms is committed; at
 * the first mismatch the later candidates are discarded, their KV rolled
 * back, and decoding resumes from the committed prefix).
 * Request r's window is rows row_start[r] .. row_start[r+1]-1 (position
 * order, clamped to [0, rows)); candidates[i] is the fast path's token for
 * the position after row i, verified[i] the fixed-shape recompute's
 * (bi_sample of that row's logits with the request's seed and step).
 *   accepted[r]   = a, the number of leading windows rows that match;
 *   commit_len[r] (in: committed tokens L) out: L + a + 1 if a < w (the
 *                 recompute's token at the mismatch is committed), else
 *                 L + w; the request's KV is valid for the first
 *                 commit_len - 1 positions, later slots are overwritten;
 *   fix_token[r]  = verified[row_start[r] + a] if a < w, else -1.
 * All arrays int32 device memory; rows = length of candidates/verified.
 * ---------------------------------------------------------------------- */
int bi_verify_commit(const int32_t *candidates, const int32_t *verified,
                     int32_t rows, const int32_t *row_start, int32_t requests,
                     int32_t *accepted, int32_t *commit_len, int32_t *fix_token,
                     void *stream);

/* ------------------------------------------------------------------------
 * Element-wise steps of a Llama-style decoder layer built around the three
 * calls above.  [LLM-42] problem statement: a token's logits must come out
 * the same whether it is verified alone or grouped with other requests, so
 * every step of the forward has to be row-independent; each of these is (one
 * fixed sequence of fp32 operations and a single round-to-nearest-even bf16
 * rounding per output element).  The pages name the steps only; the formulas
 * are the standard Llama ones.  All pointers are device pointers except where
 * a call says host; nothing is allocated; errors come back as BI_ERR_* with
 * nothing enqueued.  Device-side ids and positions are not range-checked by
 * the host: out-of-range ones are handled as each call states.
 * ---------------------------------------------------------------------- */

/* Token embedding: out[m,:] = table[tokens[m],:].  tokens: [M] int32 (ids
 * outside [0, V) give a zero row).  table: [V,H] bf16.  out: [M,H] bf16.
 * Requirements: M, V, H >= 1; H % 8 == 0; 16-byte aligned table and out. */
int bi_embed(const int32_t *tokens, const bi_bf16 *table, bi_bf16 *out,
             int64_t M, int64_t V, int64_t H, void *stream);

/* Rotary position table, computed on the HOST into host arrays cos_t and
 * sin_t of max_pos * head_dim/2 floats each: angle p * theta^(-2i/head_dim)
 * in double precision for pair i, then cos and sin each rounded once to
 * fp32.  Copy both to the device for bi_rope.  Requirements: theta > 0,
 * head_dim even and >= 2, max_pos >= 1, non-null arrays. */
int bi_rope_table(double theta, int32_t head_dim, int64_t max_pos,
                  float *cos_t, float *sin_t);

/* Rotary position embedding (rotate-half pairs i, i + D/2, D = 128) of the
 * first heads*128 values of every row of x:
 *   out[m,h,i]     = bf16(x_i c - x_{i+64} s),
 *   out[m,h,i+64]  = bf16(x_{i+64} c + x_i s),  c, s of position pos[m],
 * each product rounded to fp32 before the sum.  x: rows of x_row_stride
 * elements (so a slice of a fused q|k|v row can be read in place).  out:
 * [M, heads, 128] bf16.  pos: [M] int32; positions outside [0, max_pos)
 * give zeros.  cos_t, sin_t: device copies of the bi_rope_table arrays.
 * Requirements: M, heads >= 1; head_dim == 128; x_row_stride >= heads*128
 * and a multiple of 4; x and out 8-byte aligned; cos_t, sin_t 16-byte
 * aligned. */
int bi_rope(const bi_bf16 *x, int64_t x_row_stride, bi_bf16 *out,
            const int32_t *pos, const float *cos_t, const float *sin_t,
            int64_t M, int32_t heads, int32_t head_dim, int64_t max_pos,
            void *stream);

/* KV-cache append: row m's key and value head vectors (num_kv_heads of 128
 * each, rows k_row_stride / v_row_stride elements apart) are copied to slot
 * pos[m] % page_size of page block_table[m][pos[m] / page_size] of the
 * [num_pages][2][num_kv_heads][page_size][128] cache that
 * bi_paged_decode_attn reads.  block_table: [M, max_blocks] int32, one row
 * per appended row.  Rows whose page is negative or >= num_pages are
 * skipped.  Two rows must not name the same slot (they would race).
 * Requirements: head_dim == 128; page_size == 16; strides multiples of 8;
 * 16-byte aligned k, v and kv_pages. */
int bi_kv_append(const bi_bf16 *k, int64_t k_row_stride, const bi_bf16 *v,
                 int64_t v_row_stride, bi_bf16 *kv_pages,
                 const int32_t *block_table, const int32_t *pos, int64_t M,
                 int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                 int32_t max_blocks, int64_t num_pages, void *stream);

/* SiLU-gated product of an up projection laid out [gate | up]:
 *   out[m,f] = bf16( (g / (1 + exp(-g))) * u ),  g = gu[m,f], u = gu[m,F+f],
 * in fp32 (device exp, IEEE division).  gu: [M, 2F] bf16; out: [M, F] bf16.
 * Requirements: M, F >= 1; F % 8 == 0; 16-byte aligned gu and out. */
int bi_silu_mul(const bi_bf16 *gu, bi_bf16 *out, int64_t M, int64_t F,
                void *stream);

/* Residual add: out = bf16(a + b), one fp32 addition per element.  n values;
 * out may alias a or b.  Requirements: n >= 1; n % 8 == 0; 16-byte aligned. */
int bi_add(const bi_bf16 *a, const bi_bf16 *b, bi_bf16 *out, int64_t n,
           void *stream);

/* ------------------------------------------------------------------------
 * Measurement helper (no operation's path uses it): a matrix-core-only loop
 * that lets a benchmark quote the bf16 rate the chip sustains beside the
 * published peak.  Each of `workgroups` workgroups of 4 waves runs `iters`
 * rounds of 8 independent v_mfma_f32_16x16x32_bf16 ops per wave (16384
 * flops each) on register operands, then writes one float per lane to
 * out[workgroups * 256] (device memory, 4-byte aligned).  So one call does
 * workgroups * 4 * iters * 8 * 16384 flops.  1 <= iters <= 2^30,
 * 1 <= workgroups <= 65535.
 * ---------------------------------------------------------------------- */
int bi_ceiling_mfma(float *out, int64_t iters, int64_t workgroups,
                    void *stream);

/* Measurement helper (no operation's path uses it): a streaming read of one
 * device buffer, so that a benchmark can set a bandwidth-bound kernel beside
 * the time the same bytes take to arrive with nothing else to do.  Every
 * 16-byte chunk of p[0 .. bytes) is loaded once (consecutive lanes on
 * consecutive chunks), the words are XOR-ed together per wave, and wave w of
 * workgroup b writes out[4 b + w].  At most BI_CEILING_READ_OUT_WORDS / 4
 * workgroups run, so out must hold BI_CEILING_READ_OUT_WORDS words (device
 * memory, 4-byte aligned); words past the launch's workgroups are not
 * written.  p is read only.  Requirements: 1 <= bytes <= 2^40, bytes % 16
 * == 0, p 16-byte aligned.  Status: BI_ERR_NULL for a null p or out,
 * BI_ERR_SHAPE for a size out of range, BI_ERR_UNSUPPORTED for alignment. */
#define BI_CEILING_READ_OUT_WORDS 8192
int bi_ceiling_read(const void *p, int64_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BI_H */
