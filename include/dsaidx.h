/*
 * dsaidx.h -- C-ABI of the MI355X (gfx950) DSA lightning-indexer hot path.
 *
 * The path: quantize the per-token indexer query and the LayerNorm'd indexer key to
 * MXFP4 (E2M1 values, one UE8M0 scale per 32) or FP8 E4M3 (one power-of-two scale),
 * insert the keys into a paged cache, score every query row against its request's
 * paged keys as sum_h w[h] * ReLU(q_h . k), and select each row's top-k keys.
 *
 * Sources (documentation pages):
 *   [idx]    vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index
 *            (module text; quantize_fp4_query; DsaIndex.fp8_query; mxfp4_scale;
 *             e2m1x2; insert_key; insert_fp4_key; fp4_query_views)
 *   [fp4ops] vllm.models.kimi_k3.amd.ops.fp4_indexer
 *            (cache_views; decode_layout; quantize_queries; score_paged; store_keys)
 *   [ovl]    vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.overlap
 *            (module text: the indexer path is scoring and top-k)
 *
 * Conventions for every call:
 *  - Pointers named as device pointers must point to device memory on the current
 *    HIP device; the caller owns all of it. No call allocates, frees or reads device
 *    memory from the host, and none synchronizes: work is enqueued on `stream` (a
 *    hipStream_t; NULL is the null stream) and the call returns.
 *  - Arguments are checked on the host before anything is enqueued; a failing check
 *    returns a non-zero dsaidx_status and enqueues nothing. Conditions that could only
 *    be checked by reading device memory are caller contract and are listed per call.
 *  - Strides of typed arrays are in elements; strides of byte buffers are in bytes.
 *  - BF16 values are passed as raw 16-bit patterns.
 *  - Calls on one stream are ordered; calls that write the same memory from several
 *    streams without ordering race.
 */
#ifndef DSAIDX_H_
#define DSAIDX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSAIDX_OK = 0,
    DSAIDX_EINVAL = 1,      /* a count, size, pointer or scalar argument is invalid */
    DSAIDX_ELAYOUT = 2,     /* a stride, alignment or buffer layout breaks the required layout */
    DSAIDX_EUNSUPPORTED = 3,/* a valid shape this build does not implement (heads, max_query_len) */
    DSAIDX_EHIP = 4,        /* the HIP runtime reported an error when enqueuing */
    DSAIDX_ESCRATCH = 5     /* the sizes need more than the allocation-free call's static
                               scratch (DSAIDX_STATIC_SCRATCH_BYTES) */
} dsaidx_status;

typedef enum {
    DSAIDX_MXFP4 = 0,       /* E2M1 payload + UE8M0 scale per 32 values */
    DSAIDX_FP8 = 1,         /* E4M3FN payload + one power-of-two scale per 128 values */
    DSAIDX_FP8_MX = 2       /* as DSAIDX_FP8, the key scale stored as 4 equal UE8M0 bytes
                               ([idx] module text, insert_key with mx); queries as FP8 */
} dsaidx_format;

#define DSAIDX_DIM 128                 /* values per head and per key */
#define DSAIDX_PAGE_TOKENS 64          /* tokens per cache page */
#define DSAIDX_MXFP4_SECTION_BYTES 4352 /* [64 x 64 B E2M1 | 64 x 4 B UE8M0] */
#define DSAIDX_FP8_SECTION_BYTES 8448   /* [64 x 128 B E4M3 | 64 x 4 B scale] (also mx) */
#define DSAIDX_MAX_QUERY_LEN 16        /* query rows per request that score_paged accepts */
#define DSAIDX_TOPK_MAX_WIDTH 33554432 /* 2^25: keys per row that topk accepts */

/* Text of a status code (static storage; never NULL). */
const char *dsaidx_status_string(int status);

/* Bytes of one quantized query row: heads * 68 (MXFP4) or heads * 128 (FP8); 0 if the
 * format or head count is invalid. */
int64_t dsaidx_query_row_bytes(int fmt, int32_t heads);

/*
 * quantize_queries -- [idx] quantize_fp4_query and DsaIndex.fp8_query; [fp4ops]
 * quantize_queries (shape rules). One workgroup per row.
 *
 *  q        device, BF16 [rows, heads, 128]: element (r, h, i) at q[r*q_row_stride +
 *           h*q_head_stride + i]. Heads of 128 contiguous values; 16-byte aligned;
 *           both strides multiples of 8; q_head_stride >= 128.
 *  heads    16, 32 or 64 (DSAIDX_EUNSUPPORTED otherwise).
 *  wv       device, BF16 raw head weights [rows, heads] (unit head stride), or NULL:
 *           then w_out is not written.
 *  q_out    device bytes, row r at q_out + r*q_out_row_stride (16-byte aligned,
 *           stride a multiple of 16, >= dsaidx_query_row_bytes).
 *           MXFP4 row: [heads x 64 B E2M1 | heads x 4 B UE8M0]. Byte h*64 + j holds
 *           columns 2j (low nibble) and 2j+1 (high nibble) of head h; byte
 *           heads*64 + h*4 + g is the UE8M0 scale of columns [32g, 32g+32):
 *           e = the smallest integer with 6 * 2^e >= max(amax, 6 * 2^-126)
 *           ([idx] mxfp4_scale, read exactly), value E2M1_RNE_satfinite(v * 2^-e).
 *           FP8 row: [heads x 128 B E4M3FN]: s_h = pow2_ceil(max(1e-10, amax_h) / 448),
 *           value E4M3_RNE_satfinite(v * (1 / s_h)).
 *  w_out    device, BF16 [rows, heads]: MXFP4 BF16(wv * c_H) (the MX scales stay inside
 *           the contraction, [idx] module text); FP8 BF16((wv * s_h) * c_H)
 *           ([idx] DsaIndex.fp8_query); c_H = FP32((heads * 128)^-1/2).
 *  rows == 0 enqueues nothing and returns DSAIDX_OK.
 */
dsaidx_status dsaidx_quantize_queries(int fmt, const void *q, int64_t rows, int32_t heads,
                                      int64_t q_row_stride, int64_t q_head_stride,
                                      const void *wv, int64_t wv_row_stride, void *q_out,
                                      int64_t q_out_row_stride, void *w_out,
                                      int64_t w_out_row_stride, void *stream);

/*
 * store_keys -- [idx] insert_key, insert_fp4_key; [fp4ops] store_keys, cache_views.
 * One wavefront per key.
 *
 *  keys     device, BF16 pre-norm keys [tokens, 128], row t at keys + t*k_row_stride
 *           (4-byte aligned, k_row_stride even and >= 128).
 *  gamma, beta  device, FP32 [128] LayerNorm weight and bias (8-byte aligned).
 *  eps      LayerNorm epsilon (finite, >= 0).
 *  slots    device, int64 [tokens]: slot = page * 64 + offset. A negative slot is
 *           padding and writes nothing; a slot >= num_pages * 64 writes nothing.
 *  cache    device bytes: the section of page p starts at cache + p * page_stride
 *           (16-byte aligned; page_stride a multiple of 16 and >= the section size,
 *           4352 for MXFP4, 8448 for FP8). Only section bytes are written, so a
 *           section may live inside a larger merged page.
 *           LayerNorm: FP32, mean and variance over 128 values summed in a fixed
 *           pairwise tree, rstd = 1 / sqrt(var + eps) (IEEE), y = ((x - mean) * rstd) *
 *           gamma + beta, then rounded to BF16. MXFP4: the token's 64 payload bytes at
 *           section + offset*64, its 4 UE8M0 bytes at section + 4096 + offset*4.
 *           FP8: 128 E4M3 bytes at section + offset*128 with s = pow2_ceil(max(1e-10,
 *           amax) / 448); FP32 s at section + 8192 + offset*4 (DSAIDX_FP8_MX: the four
 *           bytes there each hold log2(s) + 127).
 *  Caller contract: slots unique within one call (duplicates race).
 *  tokens == 0 enqueues nothing.
 */
dsaidx_status dsaidx_store_keys(int fmt, const void *keys, int64_t tokens, int64_t k_row_stride,
                                const float *gamma, const float *beta, float eps,
                                const int64_t *slots, void *cache, int64_t num_pages,
                                int64_t page_stride, void *stream);

/*
 * index_inputs -- [idx] DsaIndex: the indexer inputs of one step in one launch, one
 * workgroup per token. For token t it does what dsaidx_quantize_queries does for row t of
 * q (with the raw head weights taken from the packed projection row) and what
 * dsaidx_store_keys does for the key held in the same packed row; the results are
 * bit-identical to those two calls.
 *
 *  projected  device, BF16 packed projection rows [tokens, >= proj_row_stride]: row t at
 *           projected + t*proj_row_stride (4-byte aligned, stride even); the token's
 *           pre-norm key is columns [key_col, key_col + 128) (key_col even) and its raw
 *           head weights columns [weight_col, weight_col + heads). Both ranges must lie
 *           inside the row stride. No other column is read.
 *  q, heads, q_row_stride, q_head_stride, q_out, q_out_row_stride  as in
 *           dsaidx_quantize_queries, one row per token.
 *  w_out    device, BF16 [tokens, heads] (required), as in dsaidx_quantize_queries.
 *  gamma, beta, eps, slots, cache, num_pages, page_stride  as in dsaidx_store_keys, one
 *           slot per token (negative: padding, no insert).
 *  Errors: as the two calls it combines; key_col or weight_col < 0 gives DSAIDX_EINVAL.
 *  tokens == 0 enqueues nothing.
 */
dsaidx_status dsaidx_index_inputs(int fmt, const void *projected, int64_t tokens,
                                  int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
                                  const void *q, int32_t heads, int64_t q_row_stride,
                                  int64_t q_head_stride, const float *gamma, const float *beta,
                                  float eps, const int64_t *slots, void *cache,
                                  int64_t num_pages, int64_t page_stride, void *q_out,
                                  int64_t q_out_row_stride, void *w_out, int64_t w_out_row_stride,
                                  void *stream);

/*
 * index_inputs_layout -- dsaidx_index_inputs and dsaidx_decode_layout in one launch (one more
 * workgroup computes the row bounds): the step's query / weight / key inputs and its row
 * bounds, bit-identical to the two calls. All arguments as in those two calls; the layout
 * runs even when tokens == 0. Errors: as either call.
 */
dsaidx_status dsaidx_index_inputs_layout(
    int fmt, const void *projected, int64_t tokens, int64_t proj_row_stride, int64_t key_col,
    int64_t weight_col, const void *q, int32_t heads, int64_t q_row_stride,
    int64_t q_head_stride, const float *gamma, const float *beta, float eps,
    const int64_t *slots, void *cache, int64_t num_pages, int64_t page_stride, void *q_out,
    int64_t q_out_row_stride, void *w_out, int64_t w_out_row_stride, const int32_t *seq_lens,
    const int32_t *query_lens, int64_t num_requests, int64_t num_rows, int32_t dcp_rank,
    int32_t dcp_world_size, int32_t interleave, int32_t *query_starts, int32_t *row_ends,
    void *stream);

/*
 * decode_layout -- [fp4ops] decode_layout. One workgroup; no device-to-host reads.
 *
 *  seq_lens, query_lens  device, int32 [num_requests] (query_lens >= 0).
 *  query_starts device, int32 [num_requests + 1] = [0, cumsum(query_lens)].
 *  row_ends     device, int32 [num_rows]: row r belongs to the request with
 *               query_starts[q] <= r < query_starts[q + 1] (the last request if none);
 *               end = max(0, seq - qlen + r - start + 1); rows at or past
 *               query_starts[num_requests] are graph padding with end 0. With
 *               dcp_world_size > 1 the bound is mapped to rank dcp_rank's share of keys
 *               interleaved across ranks in runs of `interleave`.
 *  Errors: num_rows < 0, num_requests < 0, dcp_rank outside [0, dcp_world_size) or
 *  interleave < 1 give DSAIDX_EINVAL.
 */
dsaidx_status dsaidx_decode_layout(const int32_t *seq_lens, const int32_t *query_lens,
                                   int64_t num_requests, int64_t num_rows, int32_t dcp_rank,
                                   int32_t dcp_world_size, int32_t interleave,
                                   int32_t *query_starts, int32_t *row_ends, void *stream);

/*
 * score_paged -- [fp4ops] score_paged (shared-key row groups, physical page strides);
 * [idx] module text (MX scales inside the logits contraction, head weights carry only
 * the weight scale). Scaled FP4 / FP8 MFMA.
 *
 *  q        device bytes: quantized query rows as written by dsaidx_quantize_queries,
 *           row r at q + r*q_row_stride (16-byte aligned, stride a multiple of 16).
 *  w        device, BF16 head weights [num_rows, heads] (w_out of quantize_queries),
 *           8-byte aligned, w_row_stride a multiple of 4.
 *  cache    device bytes, sections as for store_keys.
 *  block_table  device, int32 [num_requests, max_blocks] with row stride max_blocks:
 *           key p of request q lives on page block_table[q, p / 64], token p % 64.
 *  query_starts device, int32 [num_requests + 1]; row_ends device, int32 [num_rows]
 *           (as written by dsaidx_decode_layout).
 *  logits   device, FP32 [num_rows, max_blocks * 64], row stride >= max_blocks * 64:
 *           logits[r, p] = sum_h w[r, h] * max(0, dot_h(r, p)) for every row r of a
 *           request and every p < min(row_ends[r], max_blocks * 64), where
 *           MXFP4: dot_h = sum_g 2^(eq_g + ek_g) * sum_{i in block g} E2M1(q) * E2M1(k),
 *           FP8:   dot_h = s_k * sum_i E4M3(q) * E4M3(k).
 *           Entries at or past a row's bound, and rows of no request, are not written.
 *  max_query_len  1..16: the most rows any request has.
 *  Caller contract: query_starts nondecreasing; every request has at most
 *  max_query_len rows (further rows are not scored); block-table entries a row's
 *  bound reaches lie in [0, num_pages) (keys on other pages are not written).
 *  num_rows, num_requests or max_blocks == 0 enqueues nothing.
 */
dsaidx_status dsaidx_score_paged(int fmt, const void *q, int64_t q_row_stride, int32_t heads,
                                 const void *w, int64_t w_row_stride, const void *cache,
                                 int64_t num_pages, int64_t page_stride,
                                 const int32_t *block_table, int64_t num_requests,
                                 int64_t max_blocks, const int32_t *query_starts,
                                 const int32_t *row_ends, int64_t num_rows,
                                 int32_t max_query_len, float *logits,
                                 int64_t logits_row_stride, void *stream);

/*
 * Scoring and selection with one pass fewer over the logits ([ovl] module text: the indexer
 * path is scoring and then top-k; [fp4ops] decode_tile_size sizes logits plus selection
 * scratch together). dsaidx_score_paged_hist scores exactly as dsaidx_score_paged does (the
 * same logits, bit for bit) and also counts every written logit into a histogram per
 * (row, scoring workgroup) inside a top-k workspace; dsaidx_topk_scored then selects as
 * dsaidx_topk does (the same index sets) without its own histogram pass.
 *
 * dsaidx_score_topk_workspace_bytes: device workspace bytes for these sizes on the current
 * device (the segment geometry depends on its compute-unit count); 0 if the sizes are
 * invalid or a row would span more than 1024 scoring workgroups (more than 4,194,304 keys).
 */
size_t dsaidx_score_topk_workspace_bytes(int64_t num_requests, int64_t max_blocks,
                                         int64_t num_rows);

/*
 * dsaidx_score_segment_keys: keys per segment of those histograms (the keys one scoring
 * workgroup covers: segment s of a row holds key positions [s * n, (s + 1) * n)) for these
 * sizes on the current device; 0 if the sizes are invalid.
 */
int64_t dsaidx_score_segment_keys(int64_t num_requests, int64_t max_blocks);

/*
 * read_sections -- a bandwidth reference for dsaidx_score_paged, not a step of the indexer
 * path: a plain read of exactly the cache bytes score_paged reads -- for every request q and
 * block b < ceil(seq_lens[q] / 64) (at most max_blocks), the section (4352 B MXFP4, 8448 B FP8)
 * of page block_table[q, b] at cache + page * page_stride; entries outside [0, num_pages) are
 * skipped -- in score_paged's grid and with its per-lane loads, but no arithmetic. Each
 * wavefront writes the XOR of the 32-bit words it read; the XOR of all of out[0..words) is
 * the XOR of every word of every section read (each once).
 *
 *  cache, num_pages, page_stride, block_table, num_requests, max_blocks  as dsaidx_score_paged.
 *  seq_lens   device, int32 [num_requests]: keys per request (negative counts as 0).
 *  out        device, uint32 [out_words], out_words >= dsaidx_read_sections_words(
 *             num_requests, max_blocks) (that many words are written, on the current device).
 *  Errors: as dsaidx_score_paged for the shared arguments; a short `out` gives DSAIDX_EINVAL.
 *  num_requests, max_blocks or num_pages == 0 enqueues nothing.
 */
int64_t dsaidx_read_sections_words(int64_t num_requests, int64_t max_blocks);
dsaidx_status dsaidx_read_sections(int fmt, const void *cache, int64_t num_pages,
                                   int64_t page_stride, const int32_t *block_table,
                                   int64_t num_requests, int64_t max_blocks,
                                   const int32_t *seq_lens, uint32_t *out, int64_t out_words,
                                   void *stream);

/*
 * read_stream -- a bandwidth reference, not a step of the indexer path: a plain contiguous
 * read of `bytes` bytes at `buf` by `workgroups` workgroups of 256 lanes (workgroup b reads
 * 32 KB at b * 32 KB and then every workgroups * 32 KB further, as 16-byte loads), each
 * wavefront writing the XOR of the 32-bit words it read to out[4 * b + wavefront].
 *
 *  buf        device, 16-byte aligned, `bytes` readable bytes (a multiple of 16).
 *  workgroups 1 .. 1,048,576.
 *  out        device, uint32 [out_words], out_words >= 4 * workgroups.
 *  Errors: DSAIDX_EINVAL for a null pointer, negative or unaligned sizes, workgroups out of
 *  range or a short `out`; bytes == 0 enqueues nothing.
 */
dsaidx_status dsaidx_read_stream(const void *buf, int64_t bytes, int32_t workgroups,
                                 uint32_t *out, int64_t out_words, void *stream);

/*
 * score_paged_hist -- dsaidx_score_paged plus the top-k segment histograms.
 *  All arguments as dsaidx_score_paged, and
 *  workspace  device, >= dsaidx_score_topk_workspace_bytes(num_requests, max_blocks,
 *           num_rows) bytes, 256-byte aligned, caller-owned, no initialisation needed.
 *  Errors: as dsaidx_score_paged; a missing or short workspace gives DSAIDX_EINVAL; more
 *  than 1024 scoring workgroups per row gives DSAIDX_EUNSUPPORTED.
 */
dsaidx_status dsaidx_score_paged_hist(int fmt, const void *q, int64_t q_row_stride,
                                      int32_t heads, const void *w, int64_t w_row_stride,
                                      const void *cache, int64_t num_pages, int64_t page_stride,
                                      const int32_t *block_table, int64_t num_requests,
                                      int64_t max_blocks, const int32_t *query_starts,
                                      const int32_t *row_ends, int64_t num_rows,
                                      int32_t max_query_len, float *logits,
                                      int64_t logits_row_stride, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * Bounded logits for verify batches ([fp4ops] decode_tile_size: logits, selection scratch and
 * queries are bounded by grouping verify rows into tiles; score_paged scores one bounded
 * query tile).
 *
 * dsaidx_decode_tile_size: rows per tile, max(32, 32 * 4 * max_model_len / row_bytes) with
 * row_bytes = 4 * width + 24 * min(topk, width) + 64 * heads + 256 (integer division): the
 * rows whose logits, selection scratch and query fit in the bytes of 32 rows of FP32 logits
 * at max_model_len keys, at least 32. Returns 0 for max_model_len < 0, width < 0, topk < 1,
 * heads < 1, or sizes above 2^40.
 *
 * dsaidx_score_topk_tiled: the rows [0, num_rows) in tiles of tile_rows consecutive rows (the
 * last may be shorter), each scored as dsaidx_score_paged_hist scores it -- the same logits,
 * bit for bit -- into `logits_tile`, then selected as dsaidx_topk_scored selects (the same
 * index sets as dsaidx_topk on those logits) into its rows of `indices`. Only one tile's
 * logits and selection scratch exist at a time: after the call `logits_tile` holds the last
 * tile's logits (row r of it is row (num_rows - 1) / tile_rows * tile_rows + r). A tile may
 * split a request's rows.
 *  Scoring arguments as dsaidx_score_paged (query rows, weights and row bounds for all rows).
 *  k, indices, indices_row_stride  as dsaidx_topk: every row's selection, -1 padded.
 *  tile_rows  >= 1, e.g. dsaidx_decode_tile_size(...).
 *  logits_tile  device, FP32 [tile_rows, >= max_blocks * 64], row stride
 *             logits_tile_row_stride; caller-owned scratch.
 *  workspace  device, >= dsaidx_score_topk_tiled_workspace_bytes(num_requests, max_blocks,
 *             tile_rows, max_query_len) bytes, 256-byte aligned, caller-owned, no
 *             initialisation needed (0 from that call: invalid sizes).
 *  Two launches per tile on `stream`. Errors: as dsaidx_score_paged and dsaidx_topk_scored;
 *  tile_rows < 1 or a missing or short workspace gives DSAIDX_EINVAL.
 */
int64_t dsaidx_decode_tile_size(int64_t max_model_len, int64_t width, int32_t topk,
                                int32_t heads);
size_t dsaidx_score_topk_tiled_workspace_bytes(int64_t num_requests, int64_t max_blocks,
                                               int64_t tile_rows, int32_t max_query_len);
dsaidx_status dsaidx_score_topk_tiled(int fmt, const void *q, int64_t q_row_stride,
                                      int32_t heads, const void *w, int64_t w_row_stride,
                                      const void *cache, int64_t num_pages, int64_t page_stride,
                                      const int32_t *block_table, int64_t num_requests,
                                      int64_t max_blocks, const int32_t *query_starts,
                                      const int32_t *row_ends, int64_t num_rows,
                                      int32_t max_query_len, int32_t k, int32_t *indices,
                                      int64_t indices_row_stride, int64_t tile_rows,
                                      float *logits_tile, int64_t logits_tile_row_stride,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * index_score_hist -- one decode or verify step's indexer inputs and its scoring in one
 * launch ([idx] DsaIndex: the quantized query, the head weights and the inserted key
 * feed the logits; [fp4ops] decode_layout for the rows). Each scoring workgroup quantizes its
 * request's query rows itself, and the wavefront that scores the page of a new key
 * normalizes, quantizes and inserts that key. The results equal those of
 * dsaidx_index_inputs_layout (dcp_world_size 1) followed by dsaidx_score_paged_hist, bit for
 * bit, when each row's key slot is the position the block table gives it: row
 * query_starts[q] + i of request q holds the key at position
 * pos = seq_lens[q] - query_lens[q] + i, token pos % 64 of page block_table[q, pos / 64].
 * dsaidx_topk_scored then selects.
 *  fmt      DSAIDX_MXFP4, DSAIDX_FP8 or DSAIDX_FP8_MX (the query quantized as
 *           dsaidx_quantize_queries does, its FP8 scale folded into the head weights).
 *  projected, proj_row_stride, key_col, weight_col, q, heads, q_row_stride, q_head_stride,
 *  gamma, beta, eps  as in dsaidx_index_inputs, one packed row and one query row per row.
 *  seq_lens, query_lens, num_requests, num_rows, query_starts, row_ends  as in
 *           dsaidx_decode_layout with dcp_world_size 1 (the two outputs are written).
 *  cache, num_pages, page_stride, block_table, max_blocks  as in dsaidx_score_paged; the
 *           cache is written too (the new keys). No quantized query rows or head weights
 *           are written: they stay on chip.
 *  max_query_len  1..4 for MXFP4, 1..2 for FP8: the most rows any request has.
 *  logits, logits_row_stride, workspace, workspace_bytes  as in dsaidx_score_paged_hist.
 *  Caller contract: every request has at most max_query_len rows (further rows get neither
 *  logits nor keys); a page that receives a new key is in no other request's block table;
 *  a key whose position is negative, at or past max_blocks * 64, or on a block-table entry
 *  outside [0, num_pages) is not inserted.
 *  Errors: as the calls it replaces; max_query_len above 4 (MXFP4) or 2 (FP8) gives
 *  DSAIDX_EUNSUPPORTED. With
 *  num_rows, num_requests, max_blocks or num_pages == 0 only the row layout is written.
 */
dsaidx_status dsaidx_index_score_hist(
    int fmt, const void *projected, int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
    const void *q, int32_t heads, int64_t q_row_stride, int64_t q_head_stride, const float *gamma,
    const float *beta, float eps, const int32_t *seq_lens, const int32_t *query_lens,
    int64_t num_requests, int64_t num_rows, int32_t max_query_len, void *cache, int64_t num_pages,
    int64_t page_stride, const int32_t *block_table, int64_t max_blocks, int32_t *query_starts,
    int32_t *row_ends, float *logits, int64_t logits_row_stride, void *workspace,
    size_t workspace_bytes, void *stream);

/*
 * index_score_topk -- one step of the indexer path with its selection: dsaidx_index_score_hist
 * followed by dsaidx_topk_scored ([idx] DsaIndex; [fp4ops] decode_layout, score_paged; [ovl]
 * module text: scoring and then top-k), with the same results (row layout, cache bytes and
 * logits bit for bit, the same index sets). Where every request has one row (max_query_len 1)
 * and every row's keys lie in one scoring workgroup (dsaidx_score_segment_keys(num_requests,
 * max_blocks) >= max_blocks * 64: short rows, or many requests), it is one launch: each
 * workgroup selects its row's top-k from its own histogram and logits, and the workspace is
 * not touched. Otherwise it is the two calls, two or three launches on `stream`.
 *  All arguments of dsaidx_index_score_hist, and
 *  k, indices, indices_row_stride  as dsaidx_topk: every row's selection (graph padding rows
 *           and rows without keys select none: -1), width max_blocks * 64.
 *  Errors: as the two calls; k < 1 gives DSAIDX_EINVAL. With num_rows, num_requests,
 *  max_blocks or num_pages == 0 only the row layout is written (as dsaidx_index_score_hist).
 */
dsaidx_status dsaidx_index_score_topk(
    int fmt, const void *projected, int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
    const void *q, int32_t heads, int64_t q_row_stride, int64_t q_head_stride, const float *gamma,
    const float *beta, float eps, const int32_t *seq_lens, const int32_t *query_lens,
    int64_t num_requests, int64_t num_rows, int32_t max_query_len, void *cache, int64_t num_pages,
    int64_t page_stride, const int32_t *block_table, int64_t max_blocks, int32_t *query_starts,
    int32_t *row_ends, float *logits, int64_t logits_row_stride, int32_t k, int32_t *indices,
    int64_t indices_row_stride, void *workspace, size_t workspace_bytes, void *stream);

/*
 * topk_scored -- the per-row top-k of logits that dsaidx_score_paged_hist has just written,
 * using its histograms. Rows, bounds and output as dsaidx_topk with width = max_blocks * 64.
 *  num_requests, max_blocks, workspace  exactly as passed to the dsaidx_score_paged_hist call
 *           that wrote the logits and histograms (same stream, ordered after it; the same
 *           device). A row whose keys that call did not score (a row beyond max_query_len
 *           of its request, or keys on block-table entries outside the cache) gets
 *           unspecified positions, as its logits are unwritten; even then nothing is written
 *           at or past column k of any row.
 *  Errors: k < 1 or negative sizes give DSAIDX_EINVAL, as do num_requests or max_blocks of
 *  0 with rows to select; a short workspace gives DSAIDX_EINVAL.
 */
dsaidx_status dsaidx_topk_scored(const float *logits, int64_t num_rows, int64_t logits_row_stride,
                                 const int32_t *row_ends, int32_t k, int32_t *indices,
                                 int64_t indices_row_stride, int64_t num_requests,
                                 int64_t max_blocks, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Device workspace bytes that dsaidx_topk needs for these sizes (0: none). */
size_t dsaidx_topk_workspace_bytes(int64_t rows, int64_t width, int32_t k);

/*
 * topk -- per-row selection of the scored keys ([ovl] module text: the indexer path is
 * scoring and top-k).
 *
 *  logits   device, FP32 [rows, >= width], row stride logits_row_stride >= width.
 *  row_ends device, int32 [rows]: row r selects among positions [0, min(row_ends[r], width)).
 *  indices  device, int32 [rows, >= k], row stride >= k: the positions of the k largest
 *           logits (ties to the lower position; -0 equals +0); the order within a row is
 *           unspecified; if fewer than k positions exist, all of them and -1 after.
 *  workspace  device scratch of at least dsaidx_topk_workspace_bytes bytes, 256-byte
 *           aligned, owned by the caller; no initialisation is needed (each call writes
 *           every field before reading it). Calls that share a workspace must be ordered
 *           (one stream).
 *  Errors: k < 1, rows < 0 or width < 0 give DSAIDX_EINVAL; width above
 *  DSAIDX_TOPK_MAX_WIDTH gives DSAIDX_EUNSUPPORTED; a missing or short workspace gives
 *  DSAIDX_EINVAL. NaN logits are unsupported.
 */
dsaidx_status dsaidx_topk(const float *logits, int64_t rows, int64_t width,
                          int64_t logits_row_stride, const int32_t *row_ends, int32_t k,
                          int32_t *indices, int64_t indices_row_stride, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * topk_noalloc -- dsaidx_topk for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same selection,
 * the same index sets, with the workspace taken from a static device array of
 * DSAIDX_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on each device it runs on until
 * the process ends, instead of a caller-supplied one. It calls no hipMalloc, hipFree or other
 * allocating routine; its first call on a device looks up that device's array address (with
 * the device current) and keeps it.
 *
 *  Arguments as dsaidx_topk, without the workspace.
 *  Errors: as dsaidx_topk; sizes for which dsaidx_topk_workspace_bytes exceeds
 *  DSAIDX_STATIC_SCRATCH_BYTES give DSAIDX_ESCRATCH (nothing enqueued).
 *  Every call on a device shares that device's array, which keeps the last call's contents
 *  (the selection writes every workspace field it reads, so nothing needs clearing): calls
 *  that may overlap on one device (different streams, or different threads) race; order them
 *  on one stream.
 */
#define DSAIDX_STATIC_SCRATCH_BYTES (64ull << 20)
dsaidx_status dsaidx_topk_noalloc(const float *logits, int64_t rows, int64_t width,
                                  int64_t logits_row_stride, const int32_t *row_ends, int32_t k,
                                  int32_t *indices, int64_t indices_row_stride, void *stream);

/*
 * Decode context parallelism (DCP): [fp4ops] decode_layout deals a request's keys to W ranks
 * in runs of `interleave` (run j to rank j % W as that rank's run j / W; rank-local key
 * positions keep the global order); each rank scores and selects over its own keys with the
 * rank-local bounds dsaidx_decode_layout writes for it. [ovl] module text: the indexer path
 * then ends in a top-k merge and the local slots. The exchange between ranks (an all-gather of
 * the candidates) is the caller's; these two calls are the per-GPU parts around it.
 *
 * dcp_candidates -- one rank's merge candidates from its local top-k.
 *  logits, rows, width, logits_row_stride  the rank's local logits (as for dsaidx_topk).
 *  indices  device, int32 [rows, >= k]: the rank's local top-k positions (-1 = none).
 *  values   device, FP32 [rows, k] contiguous: logits[row, indices[row, j]] (-inf for none).
 *  positions device, int32 [rows, k] contiguous: the global key position of each candidate
 *           (-1 for none). The two outputs are this rank's slice of the gathered buffers.
 *  Errors: rows < 0, width < 0, k < 1, interleave < 1, or dcp_rank outside
 *  [0, dcp_world_size) give DSAIDX_EINVAL; global positions beyond INT32_MAX give
 *  DSAIDX_EUNSUPPORTED.
 */
dsaidx_status dsaidx_dcp_candidates(const float *logits, int64_t rows, int64_t width,
                                    int64_t logits_row_stride, const int32_t *indices, int32_t k,
                                    int64_t indices_row_stride, int32_t dcp_rank,
                                    int32_t dcp_world_size, int32_t interleave, float *values,
                                    int32_t *positions, void *stream);

/*
 * dcp_merge -- the global top-k of every row from all ranks' candidates.
 *  values, positions  device, FP32 / int32 [dcp_world_size, rows, kc] contiguous (every
 *           rank's dsaidx_dcp_candidates output, gathered; position -1 = none). Positions
 *           must be distinct within a row.
 *  merged   device, int32 [rows, >= k]: the global positions of the k largest values, ties
 *           to the lower global position (-0 equals +0); fewer than k candidates give all of
 *           them and -1 after; order within a row unspecified. When each rank's candidates
 *           are its local top-k (k each), this is the top-k over the whole row.
 *  local_slots  device, int32 [rows, >= k], or NULL: the rank-local positions of the merged
 *           keys that rank dcp_rank owns, -1 after (order unspecified).
 *  Errors: rows < 0, kc < 1, k < 1, interleave < 1, or (with local_slots) dcp_rank outside
 *  [0, dcp_world_size) give DSAIDX_EINVAL; dcp_world_size * kc > 16384 gives
 *  DSAIDX_EUNSUPPORTED.
 */
dsaidx_status dsaidx_dcp_merge(const float *values, const int32_t *positions,
                               int32_t dcp_world_size, int64_t rows, int32_t kc, int32_t k,
                               int32_t *merged, int64_t merged_row_stride, int32_t dcp_rank,
                               int32_t interleave, int32_t *local_slots,
                               int64_t local_row_stride, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSAIDX_H_ */
