/*
 * csa.h -- C ABI of libcsa: CSA / HCA hybrid compressed attention on one
 * AMD Instinct MI355X (gfx950).
 *
 * Citation keys (page title, then where on the page):
 *   [R] "DeepSeek-V4 技术解读报告" (juejin.cn/post/7631898635937497134),
 *       section 2.3 (equations 9-23, 27), section 4.3 (determinism) and
 *       section 4.6 (inference framework: the heterogeneous KV cache).
 *   [A] "DeepSeek-V4：算法架构" (1zeryu.github.io/p/deepseek-v4/), code
 *       excerpts: attention Q/KV path, Sparse Attention candidate assembly,
 *       Compressor, Indexer, HCA selection rule, output projection.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every tensor argument is a DEVICE pointer to a row-major, contiguous
 *    buffer that the caller allocates and frees.  The library allocates and
 *    frees nothing, never synchronises, and keeps no mutable global state
 *    (beyond the per-device scratch of csa_index_topk_decode_noalloc).
 *  - Element types: `dtype` (CSA_F32 or CSA_BF16) applies to hidden states,
 *    weights, queries, indexer queries/weights, caches and outputs.  The
 *    position biases `ape`, the sink logits and the compressor decode state
 *    are always fp32; indices are int32 with -1 marking an empty slot;
 *    positions are int64.
 *  - Projection weights are output-major: W has shape [out_channels, d]
 *    (a linear layer's weight layout); the projection is H . W^T, i.e.
 *    the pages' H . W with W = this buffer transposed.
 *  - Overlapped compressors (ov = 1) have 2c output channels packed as
 *    [b-series | a-series]: channels [0, c) feed the NEXT block, channels
 *    [c, 2c) the block itself ([A] Compressor).
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *    and is asynchronous.  `ws` is caller-owned scratch of at least
 *    csa_workspace_bytes(...) bytes (may be NULL when that is 0).  No entry
 *    point carries state between calls in its workspace, so it needs no
 *    clearing (csa_workspace_zero_bytes returns 0 for every entry and is
 *    kept for callers written against earlier versions of this header).
 *  - Return value: CSA_OK or a negative csa_status.  All argument checks run
 *    on the host before anything is enqueued, so a failing call has no side
 *    effect.  A fault inside a kernel surfaces at the caller's next stream
 *    synchronisation.
 *  - Precision: dot products and softmax statistics accumulate in fp32;
 *    pooling, RMSNorm and RoPE run in fp32 (RoPE angles in fp64) with one
 *    rounding to `dtype` at store.  In bf16 mode the normalised query and
 *    the attention probabilities are rounded to bf16 as matrix-core operands.
 *  - Calls on one stream are ordered; concurrent calls on different streams
 *    must not share output, state or workspace buffers.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 10

typedef enum csa_status {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = -1, /* null pointer, inconsistent sizes            */
  CSA_ERR_UNSUPPORTED = -2, /* shape/dtype outside the kernels' limits     */
  CSA_ERR_WORKSPACE = -3,   /* ws_bytes below csa_workspace_bytes(...)      */
  CSA_ERR_HIP = -4          /* a HIP launch reported an error              */
} csa_status;

typedef enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1 } csa_dtype;

/* ------------------------------------------------------------------------
 * Descriptors.  Unused fields are ignored by the calls that do not need them.
 * ---------------------------------------------------------------------- */

/* Compressor ([R] eq 9-12 for CSA, eq 20-23 for HCA) and window rows. */
typedef struct csa_compress_desc {
  int64_t n;           /* prefill: tokens in H (positions 0..n-1)           */
  int32_t batch;       /* decode: sequences B                               */
  int32_t d;           /* hidden size                                       */
  int32_t c;           /* entry width (head dim), multiple of 32, <= 512    */
  int32_t m;           /* compression ratio, 1..256                          */
  int32_t overlap;     /* 0 or 1: pool 2m rows (block i-1's b-series too)   */
  int32_t dtype;       /* csa_dtype                                          */
  int32_t qk_norm;     /* 1: RMSNorm (unit weight) on each entry / window row */
  float eps;           /* RMSNorm epsilon                                    */
  int32_t rope_dims;   /* r: rotate the last r channels (0 = off; even)      */
  float rope_theta;    /* RoPE base                                          */
  int32_t n_win;       /* window ring length (slots)                         */
  int64_t max_entries; /* decode: rows per sequence in the entry cache      */
  int64_t pos0;        /* prefill: position of the first new token, a
                          multiple of m (0 = from the start; > 0 = one chunk
                          of a chunked prefill, see csa_compress_prefill)   */
} csa_compress_desc;

/* Lightning indexer + top-k ([R] eq 16-17). */
typedef struct csa_index_desc {
  int64_t n;           /* prefill: query tokens (positions 0..n-1)          */
  int32_t batch;       /* decode: sequences B                               */
  int32_t n_heads;     /* indexer heads hI: 4, 8 or 16                      */
  int32_t head_dim;    /* indexer key width cI: 64 or 128                   */
  int32_t m;           /* compression ratio of the indexer keys             */
  int32_t k;           /* top-k, 1..2048                                     */
  int32_t dtype;       /* csa_dtype of qI, wI and the keys                  */
  int64_t n_entries;   /* prefill: rows of KI; decode: cache rows per seq   */
  int32_t score_dtype; /* prefill: CSA_F32, or CSA_BF16 to select on index
                          scores rounded to bf16 ([R] section 4.4: bf16
                          index scores for a faster selector); decode:
                          CSA_F32                                           */
  int64_t t0;          /* prefill: position of query row 0 (chunked prefill;
                          0 = from the start)                               */
} csa_index_desc;

/* Shared-KV multi-query core attention with window and sink ([R] eq 18-19,
 * 27, section 2.3.3). */
typedef struct csa_attn_desc {
  int64_t n;           /* prefill: query tokens (positions 0..n-1)          */
  int32_t batch;       /* decode: sequences B                               */
  int32_t n_heads;     /* query heads nh: 8, 16, 32 or 64                    */
  int32_t c;           /* head dim = entry width: 64, 128, 256 or 512        */
  int32_t k;           /* sparse: index slots per query                      */
  int32_t m;           /* dense (HCA): compression ratio                     */
  int32_t n_win;       /* window length (uncompressed positions incl. t)    */
  int32_t dtype;       /* csa_dtype                                          */
  float scale;         /* logit scale (c^-1/2 in the workloads)              */
  int32_t qk_norm;     /* 1: RMSNorm on each query head                      */
  float eps;           /* RMSNorm epsilon                                    */
  int32_t rope_dims;   /* r: query RoPE at t, inverse RoPE of the output    */
  float rope_theta;
  int64_t n_entries;   /* prefill: rows of comp; decode: cache rows per seq */
  int64_t t0;          /* prefill: position of query row 0 (chunked prefill;
                          0 = from the start); win_kv row 0 is then position
                          max(0, t0 - n_win + 1)                            */
} csa_attn_desc;

/* ------------------------------------------------------------------------
 * Compressor
 * ---------------------------------------------------------------------- */

/* csa_compress_prefill -- [R] eq 9-12 (CSA, ov=1) / eq 20-23 (HCA, ov=0);
 * [A] Compressor prefill branch, attention wkv -> kv_norm -> RoPE path.
 *
 * For one sequence of n tokens (positions 0..n-1):
 *   C = H W_kv^T, Z = H W_z^T                       (fp32 accumulation)
 *   entry i (i < n/m, complete blocks only): per channel, softmax over the
 *     block's m logits Z+ape (plus block i-1's b-series under overlap),
 *     weighted sum of C; then RMSNorm (qk_norm), RoPE of the last r channels
 *     at position m*i, one rounding -> out_comp[i].
 *   window rows (W_win != NULL): V = H W_win^T, RMSNorm, RoPE at the token's
 *     position -> out_win[t] and/or, for the last n_win tokens, win_ring[t % n_win].
 *   state (optional): the decode state after token n-1 (see
 *     csa_compress_decode), so decoding can continue at position n.
 *
 * Chunked prefill ([R] section 4.6, prefix reuse: entries are kept up to the
 * last complete block and only the rest is recomputed): with pos0 > 0 the n
 * new tokens sit at positions pos0 .. pos0+n-1 (pos0 % m == 0, else
 * CSA_ERR_UNSUPPORTED).  Entries, window rows, ring slots and the state are
 * those of a prefill from position 0 restricted to the new tokens: out_comp
 * row i is entry pos0/m + i, out_win row t is position pos0 + t, and the
 * state continues at pos0 + n.  Under overlap, entry pos0/m pools block
 * pos0/m - 1's b-series as well, so H then has n + m rows: the m tokens at
 * positions pos0-m .. pos0-1 (the halo) first, then the new ones.
 *
 *   H        [n, d]            dtype  ([n + m, d] under overlap with pos0 > 0)
 *   W_kv     [(1+ov)c, d]      dtype
 *   W_z      [(1+ov)c, d]      dtype
 *   ape      [m, (1+ov)c]      fp32   learned position bias B (B_b | B_a)
 *   W_win    [c, d] or NULL    dtype
 *   out_comp [floor(n/m), c]   dtype  (may be NULL when n < m)
 *   out_win  [n, c] or NULL    dtype  (requires W_win)
 *   win_ring [n_win, c] or NULL dtype (requires W_win)
 *   state    csa_state_bytes(desc with batch=1) bytes or NULL, fp32
 */
int csa_compress_prefill(const csa_compress_desc* desc, const void* H, const void* W_kv,
                         const void* W_z, const float* ape, const void* W_win, void* out_comp,
                         void* out_win, void* win_ring, float* state, void* ws, size_t ws_bytes,
                         void* stream);

/* csa_compress_decode -- [A] Compressor decode branch (start_pos > 0).
 *
 * One new token per sequence b at position pos[b] (>= 0):
 *   its projected row updates the per-sequence online pooling state; when
 *   (pos+1) mod m == 0 the block i = pos/m is finished: its entry (pooled
 *   with block i-1's b-series under overlap) goes through the epilogue at
 *   position m*i and is written to cache[b][i].  With W_win, the token's
 *   window row (RMSNorm, RoPE at pos) is written to win_ring[b][pos % n_win].
 * The state is an online softmax (running max, sum and weighted sum per
 * channel) of the current block's rows, and under overlap also of its
 * b-series and of the previous block's b-series: O(c) per sequence, not the
 * raw rows.  A state freshly produced by csa_compress_prefill(n) continues
 * at pos = n; a zero-initialised state is NOT valid -- use csa_state_init.
 *
 *   h        [B, d]               dtype
 *   pos      [B]                  int64 (device)
 *   W_kv, W_z, ape, W_win         as for prefill
 *   state    [B] x csa_state_bytes/B   fp32, updated in place
 *   cache    [B, max_entries, c]  dtype, row pos/m written on emission
 *   win_ring [B, n_win, c] or NULL
 */
int csa_compress_decode(const csa_compress_desc* desc, const void* h, const int64_t* pos,
                        const void* W_kv, const void* W_z, const float* ape, const void* W_win,
                        float* state, void* cache, void* win_ring, void* ws, size_t ws_bytes,
                        void* stream);

/* Bytes of compressor decode state for desc->batch sequences (batch >= 1). */
size_t csa_state_bytes(const csa_compress_desc* desc);

/* Writes the empty state (no token seen) for desc->batch sequences. */
int csa_state_init(const csa_compress_desc* desc, float* state, void* stream);

/* ------------------------------------------------------------------------
 * Lightning indexer + top-k
 * ---------------------------------------------------------------------- */

/* csa_index_topk_prefill -- [R] eq 16-17; [A] Indexer (causal mask, top-k of
 * min(k, visible) entries, -1 padding).
 *
 * For each token t: I[t,s] = sum_h wI[t,h] * max(0, qI[t,h,:] . KI[s,:]) over
 * the visible entries s < floor((t+1)/m); idx_out[t] receives the
 * k_t = min(k, visible) indices of largest score (ties: smaller index),
 * in ascending index order, followed by k - k_t slots of -1.
 *
 *   qI      [n, hI, cI]  dtype
 *   wI      [n, hI]      dtype
 *   KI      [n_entries, cI] dtype   (n_entries >= floor(n/m) is not required;
 *                                    entries beyond n_entries are invisible)
 *   idx_out [n, k]       int32
 * With t0 > 0 (a chunk of a chunked prefill) row t is the token at position
 * t0 + t and sees s < floor((t0+t+1)/m).  When the last row sees more than
 * 16384 entries, batches of rows are scored by the same scorer into score
 * rows in the workspace and selected by the decode top-k's selector (same
 * result definition; fp32 scores only, else CSA_ERR_UNSUPPORTED).
 */
int csa_index_topk_prefill(const csa_index_desc* desc, const void* qI, const void* wI,
                           const void* KI, int32_t* idx_out, void* ws, size_t ws_bytes,
                           void* stream);

/* csa_index_topk_decode -- the same selection for one query per sequence at
 * position pos[b] over the cached keys KI_cache[b][0 .. floor((pos+1)/m)).
 *
 *   qI       [B, hI, cI]               dtype
 *   wI       [B, hI]                   dtype
 *   KI_cache [B, n_entries, cI]        dtype
 *   pos      [B]                       int64 (device)
 *   idx_out  [B, k]                    int32, ascending, -1 padded
 */
int csa_index_topk_decode(const csa_index_desc* desc, const void* qI, const void* wI,
                          const void* KI_cache, const int64_t* pos, int32_t* idx_out, void* ws,
                          size_t ws_bytes, void* stream);

/* csa_index_topk_decode_score + csa_index_topk_decode_select -- the same
 * selection as csa_index_topk_decode in two calls, so that scoring the cached
 * keys can overlap the step's compressor ([R] eq 16-17; the pages' decode
 * step emits the new entry before the indexer scores, [A] Indexer forward).
 *
 *   _score  scores the keys of the entries that exist before each sequence's
 *           position step, KI_cache[b][0 .. floor(pos[b]/m)); it reads no row
 *           that step's csa_compress_decode writes, so it may run while that
 *           call runs on another stream.
 *   _select then, after the compressor has written the step's entry (row
 *           floor(pos/m) when (pos+1) % m == 0), scores that entry and selects
 *           over all floor((pos+1)/m) visible entries into idx_out.
 *
 * Both take the same desc, qI, wI, KI_cache, pos and workspace (sized as
 * for csa_index_topk_decode); between the two the workspace is in use and no
 * other call may touch it.
 * csa_index_topk_decode runs exactly these two steps, so the two ways give
 * bitwise the same idx_out. */
int csa_index_topk_decode_score(const csa_index_desc* desc, const void* qI, const void* wI,
                                const void* KI_cache, const int64_t* pos, void* ws,
                                size_t ws_bytes, void* stream);
int csa_index_topk_decode_select(const csa_index_desc* desc, const void* qI, const void* wI,
                                 const void* KI_cache, const int64_t* pos, int32_t* idx_out,
                                 void* ws, size_t ws_bytes, void* stream);

/* csa_index_topk_decode_noalloc -- csa_index_topk_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments and result, with
 * no workspace: the scratch is a library-owned static device array of
 * csa_noalloc_scratch_bytes() (32 MiB) bytes, one per GPU, held until the
 * process ends.  A descriptor whose csa_workspace_bytes(
 * CSA_ENTRY_INDEX_TOPK_DECODE, desc) exceeds that is rejected with
 * CSA_ERR_WORKSPACE before anything is enqueued (32 sequences of 32768
 * entries need 4.4 MiB, 4 of 262144 need 4.2 MiB: about 4 B per entry).
 * The array's device address is looked up on the first call on each device
 * (CSA_ERR_HIP if that fails).  Every call on a GPU shares the array, so
 * calls that overlap on one GPU (unordered streams, or host threads racing
 * on different streams) race; calls ordered on one stream do not.  The
 * library allocates nothing and calls no allocator. */
int csa_index_topk_decode_noalloc(const csa_index_desc* desc, const void* qI, const void* wI,
                                  const void* KI_cache, const int64_t* pos, int32_t* idx_out,
                                  void* stream);

/* Bytes of the per-device scratch csa_index_topk_decode_noalloc runs in. */
size_t csa_noalloc_scratch_bytes(void);

/* ------------------------------------------------------------------------
 * The quantised indexer path: rotation + FP4 ([A] Compressor with rotate =
 * True and the Indexer forward: rotate_activation, fp4_act_quant; [R]
 * section 4.4: the indexer QK path cached, loaded and multiplied in FP4)
 * ---------------------------------------------------------------------- */

typedef struct {
  int64_t rows;       /* rows to quantise                                      */
  int32_t width;      /* row width: 64 or 128                                  */
  int32_t dtype;      /* csa_dtype of the input                                */
} csa_fp4_desc;

/* csa_indexer_fp4_quant -- each row x[r] (width W) is rotated by the
 * normalised Walsh-Hadamard transform (x . H_W / sqrt(W), H_W the Sylvester
 * matrix) and stored in FP4: every block of 32 consecutive rotated values
 * has a scale 2^e, e the smallest integer with max|x| <= 6 * 2^e (0 for an
 * all-zero block), and each value is rounded to the nearest E2M1 value
 * (0, 0.5, 1, 1.5, 2, 3, 4, 6 times the scale, with sign), ties to the even
 * mantissa; a zero keeps no sign.
 *
 *   x      [rows, W]     dtype
 *   codes  [rows, W/2]   uint8: element 2j in the low nibble, 2j+1 in the
 *                        high one; nibble = sign << 3 | E2M1 index
 *   exps   [rows, W/32]  uint8: e + 127 per block
 * Used for the indexer keys (after their compressor) and for q^I. */
int csa_indexer_fp4_quant(const csa_fp4_desc* desc, const void* x, uint8_t* codes, uint8_t* exps,
                          void* stream);

/* csa_indexer_fp4_quant_decode -- the same rotation and FP4 for the entry a
 * decode step has just emitted into a bf16/fp32 key cache: for each of the
 * desc->rows sequences b with (pos[b] + 1) % m == 0, row pos[b] / m of
 * cache[b] ([B, n_entries, W], the csa_compress_decode output) is written to
 * row pos[b] / m of codes [B, n_entries, W/2] and exps [B, n_entries, W/32];
 * other rows are left as they are. */
int csa_indexer_fp4_quant_decode(const csa_fp4_desc* desc, const void* cache, int64_t n_entries,
                                 const int64_t* pos, int m, uint8_t* codes, uint8_t* exps,
                                 void* stream);

/* csa_index_topk_decode_fp4 -- csa_index_topk_decode on the quantised path:
 * q^I and the cached keys in the format csa_indexer_fp4_quant writes (the
 * scores are eq 16 on the dequantised values, in fp32), wI as before in
 * desc->dtype (CSA_BF16 only).  Same descriptor (head_dim = W), same
 * workspace as csa_index_topk_decode (CSA_ENTRY_INDEX_TOPK_DECODE_FP4
 * gives its size).
 *
 *   qI_codes [B, hI, cI/2], qI_exps [B, hI, cI/32]
 *   K_codes  [B, n_entries, cI/2], K_exps [B, n_entries, cI/32]
 *   wI [B, hI], pos [B], idx_out [B, k] as in csa_index_topk_decode
 * qI_codes and K_codes start on a 16-byte boundary (else
 * CSA_ERR_INVALID_ARG, checked after the workspace): the scorer loads 16
 * code bytes at a time. */
int csa_index_topk_decode_fp4(const csa_index_desc* desc, const uint8_t* qI_codes,
                              const uint8_t* qI_exps, const void* wI, const uint8_t* K_codes,
                              const uint8_t* K_exps, const int64_t* pos, int32_t* idx_out,
                              void* ws, size_t ws_bytes, void* stream);

/* csa_index_topk_prefill_fp4 -- csa_index_topk_prefill on the quantised
 * path ([R] section 4.4: the indexer's QK path in FP4 for prefill as for
 * decode): q^I and the keys in the format csa_indexer_fp4_quant writes, the
 * products taken on the scaled E2M1 matrix instruction, the scores eq 16 on
 * the dequantised values in fp32 (or rounded to bf16 with score_dtype
 * CSA_BF16), the selection as csa_index_topk_prefill.  wI in desc->dtype
 * (CSA_BF16 only).  Rows that see more than 16384 entries are not supported
 * on this path (CSA_ERR_UNSUPPORTED).  Workspace:
 * CSA_ENTRY_INDEX_TOPK_PREFILL_FP4 (the score rows, no zero bytes).
 *
 *   qI_codes [n, hI, cI/2], qI_exps [n, hI, cI/32]
 *   K_codes  [n_entries, cI/2], K_exps [n_entries, cI/32]
 *   wI [n, hI], idx_out [n, k] as in csa_index_topk_prefill
 * qI_codes and K_codes start on a 16-byte boundary (else
 * CSA_ERR_INVALID_ARG, checked after the workspace). */
int csa_index_topk_prefill_fp4(const csa_index_desc* desc, const uint8_t* qI_codes,
                               const uint8_t* qI_exps, const void* wI, const uint8_t* K_codes,
                               const uint8_t* K_exps, int32_t* idx_out, void* ws,
                               size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Core attention
 * ---------------------------------------------------------------------- */

/* csa_sparse_mqa_prefill -- [R] eq 18-19 and 27, section 2.3.3; [A] Sparse
 * Attention (window ++ selected entries, no de-duplication) and output
 * projection's inverse RoPE.
 *
 * For token t and head h: q <- RMSNorm(q[t,h]) (qk_norm), RoPE of the last r
 * channels at t; candidates = window rows win_kv[j], max(0,t-n_win+1) <= j <= t,
 * plus comp[s] for every s = idx[t][*] >= 0; logits z = scale * q . kv;
 *   o = sum_j exp(z_j) kv_j / (sum_j exp(z_j) + exp(sink[h]))
 * then inverse RoPE of the last r channels at t -> out[t,h].
 *
 *   q      [n, nh, c]   dtype
 *   win_kv [n, c]       dtype  (window rows, already normalised/rotated)
 *   comp   [n_entries, c] dtype
 *   idx    [n, k]       int32  (entries must be < n_entries or -1)
 *   sink   [nh]         fp32
 *   out    [n, nh, c]   dtype
 * With t0 > 0 (a chunk of a chunked prefill) row t is the token at position
 * t0 + t: RoPE, the window and the visible entries follow that position, and
 * win_kv holds the window rows of positions max(0, t0-n_win+1) .. t0+n-1
 * (the previous chunk's last n_win-1 rows, then the chunk's own).
 */
int csa_sparse_mqa_prefill(const csa_attn_desc* desc, const void* q, const void* win_kv,
                           const void* comp, const int32_t* idx, const float* sink, void* out,
                           void* ws, size_t ws_bytes, void* stream);

/* csa_sparse_mqa_decode -- the same for one query per sequence at pos[b];
 * window rows come from the ring (position p in slot p % n_win), entries
 * from comp_cache[b].  Candidates are split in fixed-size chunks whose
 * partial softmax states are merged in a fixed order with the sink counted
 * once, so a sequence's result does not depend on the batch ([R] 4.3).
 *
 *   q          [B, nh, c]              dtype
 *   win_ring   [B, n_win, c]           dtype
 *   comp_cache [B, n_entries, c]       dtype
 *   idx        [B, k]                  int32
 *   pos        [B]                     int64 (device)
 *   sink [nh] fp32;  out [B, nh, c] dtype
 */
int csa_sparse_mqa_decode(const csa_attn_desc* desc, const void* q, const void* win_ring,
                          const void* comp_cache, const int32_t* idx, const int64_t* pos,
                          const float* sink, void* out, void* ws, size_t ws_bytes, void* stream);

/* hca_dense_mqa_prefill -- [R] section 2.3.2 (dense attention over every
 * compressed entry), [A] HCA selection rule: as csa_sparse_mqa_prefill with
 * the candidate entries being all s < floor((t+1)/m) (and < n_entries). */
int hca_dense_mqa_prefill(const csa_attn_desc* desc, const void* q, const void* win_kv,
                          const void* comp, const float* sink, void* out, void* ws,
                          size_t ws_bytes, void* stream);

/* hca_dense_mqa_decode -- as csa_sparse_mqa_decode with all visible entries
 * comp_cache[b][0 .. floor((pos+1)/m)). */
int hca_dense_mqa_decode(const csa_attn_desc* desc, const void* q, const void* win_ring,
                         const void* comp_cache, const int64_t* pos, const float* sink,
                         void* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Decode over paged entry caches -- [R] section 4.6: the compressed
 * ("classical") caches are handed out in pages of a fixed number of raw
 * tokens, while the window ring and the compressor state (the "state cache")
 * stay preallocated per sequence.
 *
 * Each _paged call computes exactly what its contiguous form computes (the
 * results are bit-identical) with the per-sequence cache [B, N, width]
 * replaced by a shared pool of pages:
 *   pool        [P * page_entries, width]  entry rows of all sequences
 *   page_table  [B, max_pages]  int32 (device), max_pages =
 *               ceil(N / page_entries) with N = desc->max_entries (compressor)
 *               or desc->n_entries (indexer, attention)
 *   page_entries  entries per page (>= 1); a page of 128 raw tokens holds
 *               128 / m entries (32 for m = 4, 1 for m = 128)
 * Entry e of sequence b lives in pool row
 *   page_table[b * max_pages + e / page_entries] * page_entries
 *     + e % page_entries.
 * The whole table must be readable device memory, but only the values of
 * the slots of pages holding entries that the call reads (the visible
 * entries e < min(floor((pos[b]+1)/m), N) for the indexer and dense
 * attention, the entries idx names for sparse attention) or writes (the
 * emitted entry pos[b] / m) are used; each of those must name a page of the
 * pool (0 <= id < P), the other slots may hold anything.  The library cannot
 * check ids against P: an id outside the pool reads or writes outside it.
 * Two sequences may share a page only for entries that no call writes (a
 * shared prefix).  Errors: NULL page_table or page_entries < 1 ->
 * CSA_ERR_INVALID_ARG; N > 2^31 - 1 -> CSA_ERR_UNSUPPORTED; the attention
 * calls support dtype CSA_BF16 only (CSA_ERR_UNSUPPORTED otherwise).  Workspaces are those
 * of the contiguous entry (CSA_ENTRY_COMPRESS_DECODE, _INDEX_TOPK_DECODE,
 * _SPARSE_MQA_DECODE, _DENSE_MQA_DECODE).
 * ---------------------------------------------------------------------- */
/* csa_compress_prefill_paged -- csa_compress_prefill whose entries go
 * straight into a page pool ([R] section 4.6: the classical cache is handed
 * out in pages): entry e = pos0/m + i of the call (i < floor(n/m)) is
 * written to pool row page_table[e / page_entries] * page_entries +
 * e % page_entries, bit-identical to row i of the contiguous call's
 * out_comp.  One sequence: page_table is its row [ceil(N / page_entries)]
 * with N = desc->max_entries, and (pos0 + n) / m <= N (else
 * CSA_ERR_INVALID_ARG).  The window rows, ring and state are those of the
 * contiguous call; so is the workspace (CSA_ENTRY_COMPRESS_PREFILL).  Page
 * ids are used as in the paged decode calls below (0 <= id < P, unchecked). */
int csa_compress_prefill_paged(const csa_compress_desc* desc, const void* H, const void* W_kv,
                               const void* W_z, const float* ape, const void* W_win,
                               void* comp_pool, const int32_t* page_table,
                               int32_t page_entries, void* out_win, void* win_ring, float* state,
                               void* ws, size_t ws_bytes, void* stream);

int csa_compress_decode_paged(const csa_compress_desc* desc, const void* h, const int64_t* pos,
                              const void* W_kv, const void* W_z, const float* ape,
                              const void* W_win, float* state, void* cache_pool,
                              const int32_t* page_table, int32_t page_entries, void* win_ring,
                              void* ws, size_t ws_bytes, void* stream);

int csa_index_topk_decode_paged(const csa_index_desc* desc, const void* qI, const void* wI,
                                const void* KI_pool, const int32_t* page_table,
                                int32_t page_entries, const int64_t* pos, int32_t* idx_out,
                                void* ws, size_t ws_bytes, void* stream);

int csa_sparse_mqa_decode_paged(const csa_attn_desc* desc, const void* q, const void* win_ring,
                                const void* comp_pool, const int32_t* page_table,
                                int32_t page_entries, const int32_t* idx, const int64_t* pos,
                                const float* sink, void* out, void* ws, size_t ws_bytes,
                                void* stream);

int hca_dense_mqa_decode_paged(const csa_attn_desc* desc, const void* q, const void* win_ring,
                               const void* comp_pool, const int32_t* page_table,
                               int32_t page_entries, const int64_t* pos, const float* sink,
                               void* out, void* ws, size_t ws_bytes, void* stream);

/* The FP4 indexer over paged caches: the key pool [P*page_entries, cI] and
 * the FP4 pools (codes [P*page_entries, cI/2], exps [P*page_entries, cI/32])
 * share one page table, so an entry has the same row in all three.  As
 * csa_indexer_fp4_quant_decode and csa_index_topk_decode_fp4, with rows
 * mapped as above (N = n_entries, resp. desc->n_entries). */
int csa_indexer_fp4_quant_decode_paged(const csa_fp4_desc* desc, const void* cache_pool,
                                       int64_t n_entries, const int64_t* pos, int m,
                                       uint8_t* codes_pool, uint8_t* exps_pool,
                                       const int32_t* page_table, int32_t page_entries,
                                       void* stream);

int csa_index_topk_decode_fp4_paged(const csa_index_desc* desc, const uint8_t* qI_codes,
                                    const uint8_t* qI_exps, const void* wI,
                                    const uint8_t* K_codes_pool, const uint8_t* K_exps_pool,
                                    const int32_t* page_table, int32_t page_entries,
                                    const int64_t* pos, int32_t* idx_out, void* ws,
                                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Helpers
 * ---------------------------------------------------------------------- */

typedef enum csa_entry {
  CSA_ENTRY_COMPRESS_PREFILL = 0,
  CSA_ENTRY_COMPRESS_DECODE = 1,
  CSA_ENTRY_INDEX_TOPK_PREFILL = 2,
  CSA_ENTRY_INDEX_TOPK_DECODE = 3,
  CSA_ENTRY_SPARSE_MQA_PREFILL = 4,
  CSA_ENTRY_SPARSE_MQA_DECODE = 5,
  CSA_ENTRY_DENSE_MQA_PREFILL = 6,
  CSA_ENTRY_DENSE_MQA_DECODE = 7,
  CSA_ENTRY_QUERY_PROJ = 8,
  CSA_ENTRY_OUTPUT_PROJ = 9,
  CSA_ENTRY_INDEX_TOPK_DECODE_FP4 = 10,
  CSA_ENTRY_SPARSE_MQA_BACKWARD = 11,
  CSA_ENTRY_DENSE_MQA_BACKWARD = 12,
  CSA_ENTRY_INDEX_TOPK_PREFILL_FP4 = 13
} csa_entry;

/* ------------------------------------------------------------------------
 * The layer around the four calls: query path and grouped output projection
 * ---------------------------------------------------------------------- */

typedef struct {
  int64_t n;          /* rows: tokens (prefill) or sequences (one token each) */
  int32_t d;          /* hidden size, multiple of 64                          */
  int32_t d_c;        /* query latent width, multiple of 64                   */
  int32_t n_heads;    /* attention query heads                                */
  int32_t c;          /* attention head dim                                   */
  int32_t n_heads_i;  /* indexer heads                                        */
  int32_t c_i;        /* indexer head dim                                     */
  int32_t dtype;      /* CSA_BF16 (the only one these calls take)             */
  float eps;          /* latent RMSNorm epsilon                               */
} csa_query_desc;

/* csa_query_proj -- [R] eq 13-15 and 18; [A] "Q, K, V 映射与位置编码注入"
 * excerpt (wq_a -> q_norm -> wq_b) and the Indexer's wq_b / weights_proj.
 *
 *   c^Q = RMSNorm(h . W_DQ^T) * g_q   (over the d_c latent channels; rounded
 *                                      to bf16, the operand of both up
 *                                      projections)
 *   q   = c^Q . W_UQ^T,  q^I = c^Q . W_IUQ^T,  w^I = h . W_w^T
 *
 *   H      [n, d]            bf16
 *   W_DQ   [d_c, d]          bf16 (output-major, as all weights here)
 *   g_q    [d_c]             fp32, or NULL for unit weight
 *   W_w    [n_heads_i, d]    bf16
 *   W_UQ   [n_heads*c, d_c]  bf16
 *   W_IUQ  [n_heads_i*c_i, d_c] bf16
 *   q_out  [n, n_heads, c]   bf16  (the attention calls' q: their per-head
 *                                   RMSNorm and RoPE are applied there)
 *   qI_out [n, n_heads_i, c_i] bf16
 *   wI_out [n, n_heads_i]    bf16
 * Matrix products accumulate in fp32 with one rounding at store.  The
 * workspace holds the fp32 [n, d_c + n_heads_i] first product. */
int csa_query_proj(const csa_query_desc* desc, const void* H, const void* W_DQ, const float* g_q,
                   const void* W_w, const void* W_UQ, const void* W_IUQ, void* q_out,
                   void* qI_out, void* wI_out, void* ws, size_t ws_bytes, void* stream);

typedef struct {
  int64_t n;          /* rows (tokens)                                         */
  int32_t n_heads;    /* heads of the attention output                         */
  int32_t c;          /* head dim                                              */
  int32_t groups;     /* g: n_heads*c/g must be a multiple of 64               */
  int32_t d_g;        /* per-group intermediate width; g*d_g a multiple of 64  */
  int32_t d;          /* output width (hidden size)                            */
  int32_t dtype;      /* CSA_BF16                                              */
} csa_oproj_desc;

/* csa_output_proj -- [R] section 2.3.1 (d) grouped output projection; [A]
 * "输出投影" excerpt (wo_a per group, then wo_b).
 *
 *   o     [n, n_heads, c]           bf16 (an attention call's output, already
 *                                        rotated back)
 *   wo_a  [groups, d_g, n_heads*c/groups] bf16: group j of o (channels
 *                                        [j*n_heads*c/g, (j+1)*n_heads*c/g)
 *                                        of a row) -> d_g channels
 *   wo_b  [d, groups*d_g]           bf16
 *   out   [n, d]                    bf16 = concat_j(o_j . wo_a[j]^T) . wo_b^T
 * The [n, groups*d_g] intermediate is rounded to bf16 in the workspace. */
int csa_output_proj(const csa_oproj_desc* desc, const void* o, const void* wo_a, const void* wo_b,
                    void* out, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * FP8 KV rows ([A] "Q, K, V 映射与位置编码注入" and the Compressor: act_quant of
 * kv[..., :-rd] with block size 64 -- the channels without RoPE in FP8, the
 * RoPE channels at their precision; [R] section 2.3.4: the KV cache keeps the
 * RoPE dims in BF16 and the rest in FP8).  A row of c = 512 channels whose
 * last r (a multiple of 64, r < c) carry RoPE is stored as
 *   bytes [0, c-r)           E4M3 codes of channels 0 .. c-r-1 (bit 7 sign,
 *                            bits 6..3 exponent with bias 7, bits 2..0
 *                            mantissa; exponent 0 holds m * 2^-9),
 *   bytes [c-r, c+r)         channels c-r .. c-1 as bf16,
 *   bytes [c+r, c+r+(c-r)/64) one byte e + 127 per 64-channel block: its
 *                            values are code * 2^e, with e the smallest
 *                            integer >= -117 such that max |x| <= 448 * 2^e
 *                            (the floor keeps the grid step 2^(e-9) an fp32
 *                            normal; the pages leave the range open),
 * padded with zeros to csa_kv_fp8_row_bytes(c, r) (592 for c = 512, r = 64;
 * 528 for r = 0).  Codes round x / 2^e to the nearest E4M3 value, ties to
 * the even mantissa; a value that rounds to zero keeps no sign.  Source
 * values must be finite and below 2^127 in magnitude (a block scale of 2^120
 * could otherwise round a value up to 2^128, which fp32 cannot hold).
 * ---------------------------------------------------------------------- */
typedef struct csa_kv8_desc {
  int64_t rows;        /* rows to convert (decode: sequences B)             */
  int32_t c;           /* row width: 512                                    */
  int32_t rope_dims;   /* r: channels kept in bf16 (a multiple of 64, < c)   */
  int32_t dtype;       /* csa_dtype of the source rows                       */
} csa_kv8_desc;

/* Bytes of one FP8 row (0 for an unsupported c, r). */
size_t csa_kv_fp8_row_bytes(int c, int rope_dims);

/* csa_kv_fp8_quant -- src [rows, c] (dtype) -> dst [rows, row_bytes]. */
int csa_kv_fp8_quant(const csa_kv8_desc* desc, const void* src, uint8_t* dst, void* stream);

/* csa_kv_fp8_quant_decode -- the rows a decode step wrote, one per sequence
 * b < desc->rows, from src [B, n_rows, c] to dst [B, n_rows, row_bytes]:
 * ring != 0: the window slot pos[b] % n_rows (every step); ring == 0: the
 * entry pos[b] / m, only when (pos[b] + 1) % m == 0 (the step emitted it) and
 * pos[b] / m < n_rows.  Sequences with pos < 0 are skipped. */
int csa_kv_fp8_quant_decode(const csa_kv8_desc* desc, const void* src, int64_t n_rows,
                            const int64_t* pos, int m, int ring, uint8_t* dst, void* stream);

/* csa_sparse_mqa_decode_fp8 / hca_dense_mqa_decode_fp8 -- the decode
 * attention calls over FP8 rows: the window ring [B, n_win, row_bytes] and
 * the entry cache [B, n_entries, row_bytes] in the format above, decoded
 * exactly to bf16 as they are gathered; q, sink, out, idx, pos and the
 * workspace as for the bf16 calls (same descriptor, CSA_BF16, c = 512, and
 * rope_dims equal to the rows' r). */
int csa_sparse_mqa_decode_fp8(const csa_attn_desc* desc, const void* q, const void* win_ring8,
                              const void* cache8, const int32_t* idx, const int64_t* pos,
                              const float* sink, void* out, void* ws, size_t ws_bytes,
                              void* stream);
int hca_dense_mqa_decode_fp8(const csa_attn_desc* desc, const void* q, const void* win_ring8,
                             const void* cache8, const int64_t* pos, const float* sink, void* out,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Backward of the core attention ([R] section 4.3: deterministic training;
 * the attention backward accumulates in independent per-unit buffers and
 * sums them deterministically, with no atomic adds).  The gradients are the
 * chain rule through the forward of csa_sparse_mqa_prefill /
 * hca_dense_mqa_prefill (eq 19, 27; the query RMSNorm and RoPE and the
 * output's inverse RoPE of section 2.3.3), for an upstream gradient dout of
 * their output, taken with respect to
 *   dq    [n, nh, c]   the raw queries q,
 *   dwin  [n, c]       the window rows win_kv (row t is position t),
 *   dcomp [n_e, c]     the entries comp (rows no query attends to get 0),
 *   dsink [nh]         the sink logits (fp32).
 * A row that is a candidate of several queries receives the sum of their
 * contributions.  Query tokens are split into min(256, n) contiguous blocks,
 * one workgroup each, that add into their own buffers in token order; a
 * second kernel sums the buffers in block order, so results are bitwise
 * repeatable.  The softmax statistics are recomputed (no forward state is
 * taken).  Supported: dtype CSA_F32 (every tensor fp32), c in {128, 256,
 * 512}, nh in {4, 8, 16} with 512 <= nh*c <= 2048, t0 = 0; otherwise
 * CSA_ERR_UNSUPPORTED.  The workspace (CSA_ENTRY_SPARSE_MQA_BACKWARD /
 * _DENSE_MQA_BACKWARD) holds the per-block buffers: about
 * min(256, n) * (n_e + n/min(256,n) + n_win) * c * 4 bytes; it is cleared by
 * the call itself.  q, win_kv, comp, idx, sink as for the forward call. */
int csa_sparse_mqa_backward(const csa_attn_desc* desc, const void* q, const void* win_kv,
                            const void* comp, const int32_t* idx, const float* sink,
                            const void* dout, void* dq, void* dwin, void* dcomp, float* dsink,
                            void* ws, size_t ws_bytes, void* stream);
int hca_dense_mqa_backward(const csa_attn_desc* desc, const void* q, const void* win_kv,
                           const void* comp, const float* sink, const void* dout, void* dq,
                           void* dwin, void* dcomp, float* dsink, void* ws, size_t ws_bytes,
                           void* stream);

/* Workspace bytes needed by `entry` for the descriptor `desc` (a pointer to
 * the csa_*_desc type that entry takes).  Returns 0 on a null descriptor. */
size_t csa_workspace_bytes(int entry, const void* desc);

/* Leading workspace bytes that must be zero when `entry` starts: 0 for
 * every entry of this version (no entry keeps counters in its workspace). */
size_t csa_workspace_zero_bytes(int entry, const void* desc);

/* Static text for a csa_status value. */
const char* csa_status_string(int status);

/* CSA_ABI_VERSION of the loaded library. */
int csa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
