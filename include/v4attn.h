/*
 * v4attn.h -- C ABI of libv4attn.so: CSA / HCA hybrid compressed attention
 * for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * Method sources (cited by tag):
 *   [Notes] "DeepSeek V4: Towards Highly Efficient Million Token Context
 *           Intelligence" (reading notes on the technical report):
 *           §7 CSA, §8 HCA, §9 CSA/HCA other details, §11 KV cache table.
 *   [HF]    "DeepSeek-V4: a million-token context that agents can actually
 *           use" (Hugging Face blog), section "Hybrid attention: CSA and HCA".
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every data pointer is a DEVICE pointer owned by the caller; descriptor
 *    structs (v4a_kv, v4a_idx) are HOST memory holding device pointers.
 *    The library never allocates device memory: scratch comes in through a
 *    caller-provided workspace sized by v4attn_workspace_bytes().
 *  - Calls are asynchronous and stream-ordered: kernels are enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *    without synchronising.  Device faults surface at the caller's next sync.
 *  - Arguments are validated on the host before anything is enqueued; an
 *    error return leaves no side effects.  A call with nothing to do (B == 0
 *    or Q == 0; T == 0 for the chunked compressor) returns V4A_OK without
 *    looking at its data pointers, which may then be NULL.
 *  - Positions are absolute 0-based token indices.  Compressed block i covers
 *    tokens [m*i, m*(i+1)).  A query at position p sees the n_vis(p) =
 *    min(floor((p+1)/m), cap) blocks whose tokens are all at or before p, and
 *    its window is the raw tokens max(0, p-n_win+1) .. p; p < 0 sees nothing.
 *  - All arrays are row-major and densely packed in the shapes given.
 *  - Results are deterministic, and one sequence's results do not depend on
 *    the batch size B (split counts and reduction orders are fixed by the
 *    per-query shapes only).
 *  - The library keeps no mutable global state except the thread-local HIP
 *    error of the last failed call; it is thread-safe.
 */
#ifndef V4ATTN_H
#define V4ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
typedef int32_t v4a_status;
#define V4A_OK               0
#define V4A_ERR_INVALID     (-1)  /* null / inconsistent argument             */
#define V4A_ERR_UNSUPPORTED (-2)  /* outside the supported shape/format set   */
#define V4A_ERR_WORKSPACE   (-3)  /* workspace missing or too small           */
#define V4A_ERR_HIP         (-4)  /* HIP runtime / launch error (see below)   */
#define V4A_ERR_SCRATCH     (-5)  /* beyond the fixed scratch of the          */
                                  /* allocation-free entry point              */

/* ---------------------------------------------------------------- formats */
#define V4A_F32              0  /* fp32                                        */
#define V4A_BF16             1  /* bf16 (raw 16-bit patterns)                  */
#define V4A_KV_FP8_BF16ROPE  2  /* attention entry: e4m3fn nope + bf16 RoPE +
                                   one fp32 scale per entry ([Notes §9]: RoPE
                                   dims in BF16, every other KV dim in FP8)    */
#define V4A_IDX_MXFP4        3  /* indexer key: OCP MXFP4, e2m1 elements with
                                   one e8m0 scale per 32 ([Notes §9]: the
                                   lightning indexer runs in FP4)              */

/*
 * Attention entries: a compressed cache, or a ring of raw (uncompressed)
 * tokens for the sliding-window branch.  `cap` rows per sequence; row r of
 * sequence b lives at [b][r].  For a window ring, token t lives at row t mod
 * cap.  Entry value (used as both key and value, [Notes §7] shared-KV MQA):
 *   V4A_F32:             nope f32 [B][cap][d_nope] ++ rope f32 [B][cap][d_rope]
 *   V4A_KV_FP8_BF16ROPE: nope u8 e4m3fn [B][cap][d_nope] times scale f32 [B][cap],
 *                        ++ rope bf16 [B][cap][d_rope]; scales are finite and
 *                        >= 0 (v4attn_compress writes amax / 448)
 */
typedef struct {
  int32_t fmt;      /* V4A_F32 | V4A_KV_FP8_BF16ROPE                          */
  int32_t d_nope;   /* non-RoPE dims                                           */
  int32_t d_rope;   /* RoPE dims (the last d_rope dims of the entry)           */
  int32_t _pad;
  int64_t cap;      /* rows per sequence                                       */
  void   *nope;
  void   *rope;
  float  *scale;    /* NULL for V4A_F32                                        */
} v4a_kv;

/*
 * Compressed lightning-indexer keys, `cap` rows per sequence.
 *   V4A_F32:       codes f32 [B][cap][d]
 *   V4A_IDX_MXFP4: codes u8 [B][cap][d/2] (element 2i in the LOW nibble of
 *                  byte i), scales u8 e8m0 [B][cap][d/32] (value 2^(byte-127))
 */
typedef struct {
  int32_t  fmt;     /* V4A_F32 | V4A_IDX_MXFP4                                */
  int32_t  d;
  int64_t  cap;
  void    *codes;
  uint8_t *scales;  /* NULL for V4A_F32                                        */
} v4a_idx;

/* output kinds of v4attn_compress */
#define V4A_OUT_KV   0      /* `out` points to a v4a_kv  */
#define V4A_OUT_IDX  1      /* `out` points to a v4a_idx */

/*
 * v4attn_compress -- softmax-gated token pooling ([Notes §8] HCA compressor
 * equations; [Notes §7] CSA overlap compressor; [HF] "softmax-gated pooling
 * with a learned positional bias").  For every complete block i of the call
 * and every channel c, a softmax over the block's slots of (gate + positional
 * bias), then the weighted sum of the slots' KV values:
 *   non-overlap (kv_prev == NULL): m slots, the m tokens of block i;
 *   overlap: 2m slots = the m previous-role tokens of block i-1 followed by
 *            the m current-role tokens of block i (block 0 has no previous
 *            block: only its m current slots count).
 * The pooled fp32 row is then stored in the cache's format (FP8: scale =
 * fp32(amax/448) over the d_nope dims, code = e4m3fn(x/scale) with RNE and
 * saturation; MXFP4: per 32, e = floor(log2 amax) - 2, code = e2m1(x/2^e) RNE
 * saturating; BF16 RoPE dims RNE).  With m = 1 and no overlap this is a plain
 * store/quantisation of the token rows (the window ring is filled that way).
 *
 *   kv_cur, gate_cur   [B][T][d] tokens t0 .. t0+T-1 (gate_cur NULL = all 0)
 *   kv_prev, gate_prev [B][T][d] tokens t0-m .. t0+T-m-1, or both NULL (no
 *                      overlap); with t0 == 0 the first m rows are not read
 *   pos_bias           f32 [slots][d], slots = 2m (overlap) or m; NULL = 0
 *   in_dtype           V4A_F32 | V4A_BF16 (for kv_* and gate_*)
 *   m                  1, 2, 4, ..., 128;  T and t0 multiples of m; t0 >= 0
 *   out_kind, out      V4A_OUT_KV + v4a_kv* | V4A_OUT_IDX + v4a_idx* (host);
 *                      rows (t0/m + j) mod cap, j < T/m, of every sequence
 *                      are written; nothing else is touched.  When T/m > cap
 *                      only the last cap blocks are written (the ring keeps
 *                      the newest entries).
 * Supported: d <= 1024; KV out: d == d_nope + d_rope, FP8 needs d_nope%32==0;
 * IDX out: d == out->d, MXFP4 needs d%32 == 0.
 */
v4a_status v4attn_compress(const void *kv_cur, const void *gate_cur,
                           const void *kv_prev, const void *gate_prev,
                           const float *pos_bias, int32_t in_dtype,
                           int32_t B, int32_t T, int32_t d, int32_t m,
                           int64_t t0, int32_t out_kind, const void *out,
                           void *stream);

/*
 * Query / KV-entry RMSNorm and partial RoPE ([Notes §9]: every query head and
 * every compressed KV entry is RMS-normalised before core attention; RoPE acts
 * on the last 64 dims of the query, of the KV entry and of the core-attention
 * output, which is rotated back by the query's position since an entry is
 * both key and value).
 *   RMSNorm(x) = x / sqrt(mean(x^2) + eps) * gamma over the D dims of a head
 *   or an entry.  RoPE rotates adjacent pairs (x[2i], x[2i+1]) of the last
 *   d_rope dims by a = fl32(fl32(pos) * inv_freq[i]) (one fp32 product):
 *   (x0, x1) -> (x0 cos a - x1 sin a, x0 sin a + x1 cos a).
 * Positions: a query's is pos[b][j]; a compressed entry's the last token of
 * its block (i * m + m - 1, the first position that sees it); a window
 * token's (compressed with m = 1) its own index.
 */
typedef struct {
  const float *gamma;     /* device f32 [D] RMSNorm weight, or NULL: no RMSNorm   */
  const float *inv_freq;  /* device f32 [d_rope / 2] RoPE inverse frequencies, or
                             NULL: no RoPE                                        */
  float eps;              /* RMSNorm epsilon, >= 0                                */
  int32_t _pad;
} v4a_norm_rope;

/*
 * v4attn_compress_nr -- v4attn_compress with the KV-entry RMSNorm and RoPE
 * (v4a_norm_rope, host struct holding device pointers) applied to every pooled
 * entry, in fp32, before it is stored or quantised (the FP8 scale is taken
 * after them).  KV outputs only (out_kind V4A_OUT_KV, d_nope even, d_rope
 * even); nr NULL behaves as v4attn_compress.  Errors as v4attn_compress, plus
 * V4A_ERR_UNSUPPORTED for indexer-key outputs and V4A_ERR_INVALID for eps < 0.
 */
v4a_status v4attn_compress_nr(const void *kv_cur, const void *gate_cur,
                              const void *kv_prev, const void *gate_prev,
                              const float *pos_bias, int32_t in_dtype,
                              int32_t B, int32_t T, int32_t d, int32_t m,
                              int64_t t0, int32_t out_kind, const void *out,
                              const v4a_norm_rope *nr, void *stream);

/*
 * v4attn_index_topk -- lightning indexer + top-k selector ([Notes §7]:
 * I_{t,s} = sum_h w_{t,h} ReLU(q_{t,h} . K_s), then Top-k over s).
 * For each query (b, j) at position pos[b][j], scores every visible block
 * s < n_vis(p) and returns the k' = min(k, n_vis) highest-scoring block ids
 * (ties: lower id first), listed in ascending order, padded with -1 to k.
 * With MXFP4 keys the query heads are quantised to MXFP4 (groups of 32) in the
 * call ([Notes §9]: FP4 indexer QK path); with F32 keys nothing is quantised.
 * Scores are accumulated and ranked in fp32.
 *
 *   q_idx   [B][Q][H_I][d]  dtype q_dtype (V4A_F32 | V4A_BF16)
 *   w       f32 [B][Q][H_I] head weights (any sign)
 *   keys    host v4a_idx (device arrays inside), d = keys->d
 *   pos     int64 [B][Q]
 *   topk    int32 [B][Q][k] output
 *   ws      workspace of at least v4attn_workspace_bytes(V4A_OP_INDEX_TOPK, ...)
 * Supported: MXFP4 keys with d == 128 and H_I in {16,32,48,64}; F32 keys with
 * d <= 256, H_I <= 64; 1 <= k <= 4096.
 */
v4a_status v4attn_index_topk(const void *q_idx, int32_t q_dtype, const float *w,
                             const v4a_idx *keys, const int64_t *pos,
                             int32_t B, int32_t Q, int32_t H_I, int32_t m,
                             int32_t k, int32_t *topk,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * v4attn_index_topk_noalloc -- v4attn_index_topk for callers that cannot
 * allocate device memory or own a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments
 * (minus ws / ws_bytes), results, supported set and errors as
 * v4attn_index_topk; the call's scratch (scores, histograms, candidates)
 * lives in a fixed device array of the library, 32 MiB on every GPU the
 * library runs on, held until the process ends.  The call allocates nothing
 * (no hipMalloc / hipFree); its first call on a device looks up that
 * device's copy of the array (hipGetSymbolAddress, once per device).
 *   V4A_ERR_SCRATCH  the call needs more than 32 MiB, i.e. more than
 *                    v4attn_workspace_bytes(V4A_OP_INDEX_TOPK, ...) allows
 *                    (about 1.15 MiB per query row at 262144 MXFP4
 *                    blocks: up to 27 rows B * Q at a 1M-token context);
 *                    nothing is enqueued.
 * Every call on a GPU shares that GPU's array and leaves its contents
 * behind; the kernels clear what must start at zero.  Calls that overlap on
 * one GPU (on different streams, or from different threads) race on the
 * array: the caller orders them (one stream, or events).
 */
v4a_status v4attn_index_topk_noalloc(const void *q_idx, int32_t q_dtype, const float *w,
                                     const v4a_idx *keys, const int64_t *pos,
                                     int32_t B, int32_t Q, int32_t H_I, int32_t m,
                                     int32_t k, int32_t *topk, void *stream);

/*
 * v4attn_index_topk_bf16 -- the selector variant with BF16 index scores
 * ([Notes §9]: the top-k selector's index scores go from FP32 to BF16).
 * Same arguments, workspace, supported set and errors as v4attn_index_topk;
 * each fp32 score is rounded to the nearest bf16 (ties to even) before it is
 * ranked, so scores that become equal are ordered by id (lower id first).
 * The workspace's score rows hold the bf16 values (half the traffic of the
 * fp32 scores through the selector).
 */
v4a_status v4attn_index_topk_bf16(const void *q_idx, int32_t q_dtype, const float *w,
                                  const v4a_idx *keys, const int64_t *pos,
                                  int32_t B, int32_t Q, int32_t H_I, int32_t m,
                                  int32_t k, int32_t *topk,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * v4attn_csa_attend -- CSA core attention ([Notes §7]: shared key-value MQA
 * over the selected compressed entries, plus the sliding-window branch over
 * the most recent n_win uncompressed entries; [Notes §8] table: both sets enter
 * core attention together, i.e. one joint softmax; [Notes §9]: optional
 * per-head attention sink logit).  For query (b, j) at p = pos[b][j], head h:
 *   E = { comp row s : s in topk[b][j][:], 0 <= s < comp->cap }  (ids outside
 *       [0, cap) are skipped; no de-duplication)  ++  window tokens of p
 *   l_e = sm_scale * (q_h . v_e);  out_h = sum_e softmax(l, sink_h)_e v_e
 *   (the sink adds exp(sink_h - M) to the denominator only); empty E -> 0.
 *
 *   q      [B][Q][H][D] q_dtype, D = comp->d_nope + comp->d_rope
 *   comp, win   host v4a_kv (same format and dims)
 *   topk   int32 [B][Q][k];  n_win >= 0;  pos int64 [B][Q]
 *   sink   f32 [H] or NULL
 *   out    [B][Q][H][D] out_dtype (V4A_F32 | V4A_BF16)
 * Supported: F32 entries with D <= 512, D % 8 == 0, H <= 128 (q F32 or BF16);
 * FP8 entries with d_nope == 448, d_rope == 64, q BF16, H % 16 == 0, H <= 128.
 * win->cap must be >= n_win (the caller keeps every window token of every
 * query of the call in the ring).
 */
v4a_status v4attn_csa_attend(const void *q, int32_t q_dtype, const v4a_kv *comp,
                             const int32_t *topk, int32_t k,
                             const v4a_kv *win, int32_t n_win, const int64_t *pos,
                             const float *sink, float sm_scale,
                             int32_t B, int32_t Q, int32_t H,
                             void *out, int32_t out_dtype,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * v4attn_csa_index_attend -- one CSA layer's indexer, top-k selector and
 * core attention in one call ([Notes §7]: lightning indexer, Top-k selector,
 * shared key-value MQA over the selected entries plus the sliding window;
 * [Notes §9] FP4 indexer QK, FP8 entries).  Same results as
 * v4attn_index_topk followed by v4attn_csa_attend on the same arguments
 * (bit for bit: topk and out are what the two calls write): topk is filled
 * and out is the attention over comp rows topk[b][j][:] plus the window.
 * When every row takes the three-filter selection (not the sampled one of
 * query-tiled scans) and the entries are FP8, the selector's last step
 * (ordering the selected ids) runs inside the attention kernel, one launch
 * fewer; otherwise the two calls run in sequence.
 *
 *   q_idx, q_idx_dtype, w, keys, H_I, m, k, topk   as v4attn_index_topk
 *   q, q_dtype, comp, win, n_win, sink, sm_scale, H, out, out_dtype
 *                                                  as v4attn_csa_attend
 *   pos    int64 [B][Q], the positions of both
 *   ws_index   at least v4attn_workspace_bytes(V4A_OP_CSA_INDEX, B, Q, H_I,
 *              keys->d, keys->cap, k, 0) bytes (the index workspace plus the
 *              selector's per-chunk lists, 8 bytes per key row and query)
 *   ws_attend  at least v4attn_workspace_bytes(V4A_OP_CSA_ATTEND, B, Q, H, D,
 *              0, k, n_win) bytes
 * Supported set and errors: those of the two calls; the timing events of
 * v4attn_time_next_kernel are not consumed.
 */
v4a_status v4attn_csa_index_attend(const void *q_idx, int32_t q_idx_dtype, const float *w,
                                   const v4a_idx *keys, int32_t H_I, int32_t m, int32_t k,
                                   int32_t *topk, const void *q, int32_t q_dtype,
                                   const v4a_kv *comp, const v4a_kv *win, int32_t n_win,
                                   const int64_t *pos, const float *sink, float sm_scale,
                                   int32_t B, int32_t Q, int32_t H, void *out, int32_t out_dtype,
                                   void *ws_index, size_t ws_index_bytes, void *ws_attend,
                                   size_t ws_attend_bytes, void *stream);

/*
 * v4attn_hca_attend -- HCA core attention ([Notes §8]: no top-k; dense over
 * every visible compressed entry, plus the same window branch).  As
 * v4attn_csa_attend with E = { comp rows s < n_vis(p) } ++ window tokens of p.
 */
v4a_status v4attn_hca_attend(const void *q, int32_t q_dtype, const v4a_kv *comp,
                             int32_t m, const v4a_kv *win, int32_t n_win,
                             const int64_t *pos, const float *sink, float sm_scale,
                             int32_t B, int32_t Q, int32_t H,
                             void *out, int32_t out_dtype,
                             void *ws, size_t ws_bytes, void *stream);

/*
 * v4attn_csa_attend_nr / v4attn_hca_attend_nr -- the attend calls with the
 * query RMSNorm and RoPE (v4a_norm_rope; the query's own position) applied
 * before attention, and the output's last d_rope dims rotated back by the
 * query position ([Notes §9]).  The normalised, rotated query is rounded to
 * bf16 (the attention's operand precision) inside the attention kernel; the
 * workspace is the plain call's (V4A_OP_CSA_ATTEND_NR / _HCA_ATTEND_NR size it
 * the same).
 * The cache entries are expected to carry their own RMSNorm and RoPE
 * (v4attn_compress_nr).  FP8 entries only (V4A_KV_FP8_BF16ROPE); nr NULL
 * behaves as the plain call.  Errors as the plain calls, plus
 * V4A_ERR_UNSUPPORTED for fp32 entries and V4A_ERR_INVALID for eps < 0.
 */
v4a_status v4attn_csa_attend_nr(const void *q, int32_t q_dtype, const v4a_kv *comp,
                                const int32_t *topk, int32_t k, const v4a_kv *win,
                                int32_t n_win, const int64_t *pos, const float *sink,
                                float sm_scale, int32_t B, int32_t Q, int32_t H,
                                void *out, int32_t out_dtype, const v4a_norm_rope *nr,
                                void *ws, size_t ws_bytes, void *stream);
v4a_status v4attn_hca_attend_nr(const void *q, int32_t q_dtype, const v4a_kv *comp,
                                int32_t m, const v4a_kv *win, int32_t n_win,
                                const int64_t *pos, const float *sink, float sm_scale,
                                int32_t B, int32_t Q, int32_t H,
                                void *out, int32_t out_dtype, const v4a_norm_rope *nr,
                                void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- paged cache
 * [Notes §11] KV cache table: the classical cache holds the compressed
 * entries in blocks, each covering a span of raw tokens and holding the
 * entries that span produces; the block size is a multiple of the least
 * common multiple of the two compression ratios (4 and 128, so 128 tokens),
 * so one layout serves both kinds of layer.  The state cache is a fixed-size
 * region per sequence: the sliding-window entries and the uncompressed tail
 * of the compressor block that is not full yet, updated as the position
 * advances.
 *
 * Here a block of the classical cache is a page of `page_tokens` raw tokens;
 * a layer of compression rate m keeps P = page_tokens / m entries per page.
 * A paged cache is a pool of pages, and the v4a_kv / v4a_idx of a paged call
 * describes the pool: its arrays have no batch axis, [cap][...] with cap =
 * n_pages * P pool rows.  Logical entry r of sequence b (its compressed block
 * r) is pool row table[b][r / P] * P + r % P, and a sequence holds at most
 * max_pages * P entries: that logical capacity takes the place of `cap` in
 * n_vis.  Page ids outside [0, n_pages) are clamped into it on the device, so
 * no table content addresses memory outside the pool (such a page reads or
 * writes the clamped page).  Top-k ids are logical block ids.  The window ring
 * stays a per-sequence ring (state cache), as in the plain calls.
 * Supported: page_tokens a power of two, 128 <= page_tokens <= 2^30, m <=
 * page_tokens; n_pages * P and max_pages * P below 2^31; FP8 entries
 * (V4A_KV_FP8_BF16ROPE) for attention, MXFP4 keys with P >= 128 for the
 * indexer (fp32 caches are not paged).
 */
typedef struct {
  const int32_t *table;   /* device int32 [B][max_pages]: pool page of each page */
  int32_t max_pages;      /* table row length, >= 1                           */
  int32_t page_tokens;    /* raw tokens per page                              */
} v4a_pages;

/*
 * v4attn_compress_paged -- v4attn_compress (and, with nr non-NULL, its _nr
 * form) writing block t0/m + j of sequence b to its pool row instead of a ring
 * row; t0/m + T/m must not exceed max_pages * P (V4A_ERR_INVALID).
 */
v4a_status v4attn_compress_paged(const void *kv_cur, const void *gate_cur,
                                 const void *kv_prev, const void *gate_prev,
                                 const float *pos_bias, int32_t in_dtype,
                                 int32_t B, int32_t T, int32_t d, int32_t m,
                                 int64_t t0, int32_t out_kind, const void *out,
                                 const v4a_pages *pages, const v4a_norm_rope *nr,
                                 void *stream);

/*
 * v4attn_append -- the decode-time compressor step ([Notes §11] state cache):
 * one new token per sequence.  For every b with p = pos[b] >= 0, the token's
 * rows kv_cur[b], gate_cur[b], kv_prev[b], gate_prev[b] ([B][d] each, the
 * streams of v4attn_compress; gates may be NULL = 0, kv_prev NULL = no
 * overlap) are folded into the sequence's pooling state; if p + 1 is a
 * multiple of m, the token completes block i = (p + 1) / m - 1, whose entry --
 * the value v4attn_compress gives that block (current rows: tokens i*m .. p;
 * previous-role rows: tokens (i-1)*m .. i*m - 1, none for block 0) -- is
 * stored, with nr after the entry RMSNorm and RoPE, at ring row i mod cap
 * (pages NULL) or at its pool row (pages non-NULL; a block beyond the
 * sequence's max_pages * P entries is not stored).  pos[b] < 0 leaves
 * sequence b untouched.
 *
 * The state cache of the compressor holds, instead of the raw rows of the
 * unfinished block, their running softmax pooling: state is device f32
 * [B][2][3][d] -- for the block of the current token and for the
 * previous-role part of the next block, per channel the running maximum of
 * the logits, the denominator and the numerator.  A step folds one token in,
 * and a block completes with one division (O(1) work per token).  The state
 * needs no initialisation: a token at slot 0 of its block resets the parts
 * it starts.  Calls for one sequence must come in position order with every
 * position once, and a sequence's first call must be at slot 0 of a block.
 * With out NULL the call only updates the state (nothing is stored; out_kind,
 * pages and nr are ignored): to continue after a chunked prefill of tokens
 * 0 .. P-1 (v4attn_compress over its complete blocks), first append tokens
 * max(0, m * (floor(P / m) - 1)) .. m * floor(P / m) - 1 with out NULL, then
 * every later token normally.  state may be NULL only for m == 1 without
 * overlap (the token is the whole block: the window ring is filled so).
 *
 *   state    device f32 [B][2][3][d], or NULL as above
 *   pos      int64 [B]
 *   out_kind, out, nr  as v4attn_compress_nr / _paged; out may be NULL
 * Errors: as v4attn_compress_paged; V4A_ERR_INVALID for a missing state.
 */
v4a_status v4attn_append(const void *kv_cur, const void *gate_cur,
                         const void *kv_prev, const void *gate_prev,
                         float *state, const int64_t *pos,
                         const float *pos_bias, int32_t in_dtype,
                         int32_t B, int32_t d, int32_t m,
                         int32_t out_kind, const void *out,
                         const v4a_pages *pages, const v4a_norm_rope *nr,
                         void *stream);

/*
 * v4attn_append_batch -- up to V4A_MAX_APPEND v4attn_append calls in one
 * launch (a decode step's appends of several caches: a layer's entries,
 * indexer keys and window ring, or several layers).  calls[j] holds the
 * arguments of one v4attn_append (host struct; out, pages and nr are host
 * pointers as there).  The result is that of the calls made one after the
 * other, provided no two of them write the same state or the same cache
 * rows (they run concurrently).  Every call is validated before anything
 * is launched; the first invalid one's status is returned.
 */
#define V4A_MAX_APPEND 8
typedef struct {
  const void *kv_cur, *gate_cur, *kv_prev, *gate_prev;   /* [B][d] token rows */
  float *state;                 /* f32 [B][2][3][d], or NULL (m == 1, no overlap) */
  const int64_t *pos;           /* int64 [B] */
  const float *pos_bias;        /* f32 [slots][d] or NULL */
  const void *out;              /* host v4a_kv / v4a_idx, or NULL: state only */
  const v4a_pages *pages;       /* or NULL: ring rows */
  const v4a_norm_rope *nr;      /* or NULL */
  int32_t in_dtype, B, d, m, out_kind, _pad;
} v4a_append;
v4a_status v4attn_append_batch(int32_t n, const v4a_append *calls, void *stream);

/*
 * v4attn_index_topk_paged -- v4attn_index_topk over paged MXFP4 keys (keys
 * describes the pool; P = page_tokens / m >= 128).  score_bf16 != 0 selects
 * the BF16-score ranking of v4attn_index_topk_bf16.  Workspace: as
 * V4A_OP_INDEX_TOPK with cap = max_pages * P.
 */
v4a_status v4attn_index_topk_paged(const void *q_idx, int32_t q_dtype, const float *w,
                                   const v4a_idx *keys, const v4a_pages *pages,
                                   const int64_t *pos, int32_t B, int32_t Q, int32_t H_I,
                                   int32_t m, int32_t k, int32_t score_bf16, int32_t *topk,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * v4attn_csa_attend_paged / v4attn_hca_attend_paged -- the attend calls (and,
 * with nr non-NULL, their _nr forms) over a paged compressed cache of
 * compression rate m (comp describes the pool; FP8 entries).  CSA: top-k ids
 * are logical block ids; ids outside [0, max_pages * P) are skipped.
 * Workspace: as the plain (or _nr) op, with cap = max_pages * P for HCA.
 */
v4a_status v4attn_csa_attend_paged(const void *q, int32_t q_dtype, const v4a_kv *comp,
                                   const v4a_pages *pages, int32_t m,
                                   const int32_t *topk, int32_t k, const v4a_kv *win,
                                   int32_t n_win, const int64_t *pos, const float *sink,
                                   float sm_scale, int32_t B, int32_t Q, int32_t H,
                                   void *out, int32_t out_dtype, const v4a_norm_rope *nr,
                                   void *ws, size_t ws_bytes, void *stream);
v4a_status v4attn_hca_attend_paged(const void *q, int32_t q_dtype, const v4a_kv *comp,
                                   const v4a_pages *pages, int32_t m,
                                   const v4a_kv *win, int32_t n_win, const int64_t *pos,
                                   const float *sink, float sm_scale,
                                   int32_t B, int32_t Q, int32_t H,
                                   void *out, int32_t out_dtype, const v4a_norm_rope *nr,
                                   void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------- helpers */
#define V4A_OP_INDEX_TOPK 1
#define V4A_OP_CSA_ATTEND 2
#define V4A_OP_HCA_ATTEND 3
#define V4A_OP_CSA_ATTEND_NR 4   /* the _nr variants (same sizes as the plain ops) */
#define V4A_OP_HCA_ATTEND_NR 5
#define V4A_OP_CSA_INDEX 6       /* the index workspace of v4attn_csa_index_attend */

/*
 * Workspace bytes a call needs (0 = none).  Arguments that do not apply to
 * `op` are ignored:
 *   INDEX_TOPK, CSA_INDEX: B, Q, H (= H_I), d (= key dim), cap (= keys->cap), k
 *   CSA_ATTEND(_NR): B, Q, H, d (= D), cap (ignored), k, n_win
 *   HCA_ATTEND(_NR): B, Q, H, d (= D), cap (= comp->cap), k (= m), n_win
 * Returns (size_t)-1 for an invalid combination.
 */
size_t v4attn_workspace_bytes(int32_t op, int32_t B, int32_t Q, int32_t H,
                              int32_t d, int64_t cap, int32_t k, int32_t n_win);

/* Human-readable status text (static storage). */
const char *v4attn_status_str(v4a_status s);

/* hipError_t behind the calling thread's last V4A_ERR_HIP (0 if none). */
int32_t v4attn_last_hip_error(void);

/*
 * Kernel timing (measurement helper).  The calling thread's next call of
 * v4attn_index_topk(_bf16), v4attn_csa_attend(_nr) or v4attn_hca_attend(_nr) records `start`
 * and `stop` (hipEvent_t handles created by the caller) on the call's stream
 * immediately before and after its dominant kernel -- the index scan, resp.
 * the attention kernel (not the split merge) -- so hipEventElapsedTime gives
 * that kernel's duration.  The events are consumed by that one call; NULL
 * clears them.  Calls that fail validation consume nothing.  Meant for eager
 * launches, not for stream capture.
 */
void v4attn_time_next_kernel(void *start, void *stop);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t v4attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* V4ATTN_H */
