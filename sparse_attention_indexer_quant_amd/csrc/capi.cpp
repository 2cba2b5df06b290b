// C-ABI of the indexer hot path (include/dsaidx.h): argument checks on the host, then one
// launch per call on the caller's stream. A failing check returns before any HIP call, so
// every error path can be exercised without a GPU.
//
// The checks follow the shape rules on page "vllm.models.kimi_k3.amd.ops.fp4_indexer":
// cache_views (uint8 [pages, 64, 68] sections, physical stride >= 4352), quantize_queries
// (contiguous 128-element heads; 16, 32 or 64 heads), store_keys (contiguous 128-element
// keys, one slot per key), decode_layout (DCP geometry, non-negative row count) and
// score_paged (empty outputs return at once); plus the alignments the kernels' vector
// loads and stores need.
#include <cmath>
#include <cstdint>

#include "dsaidx.h"
#include "launch.h"
#include "layout.h"
#include "topk_layout.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool valid_fmt(int fmt) { return fmt == DSAIDX_MXFP4 || fmt == DSAIDX_FP8 || fmt == DSAIDX_FP8_MX; }

bool valid_heads(int heads) { return heads == 16 || heads == 32 || heads == 64; }

int64_t section_bytes(int fmt) {
    return fmt == DSAIDX_MXFP4 ? DSAIDX_MXFP4_SECTION_BYTES : DSAIDX_FP8_SECTION_BYTES;
}

// FP32 (heads * 128)^-1/2, nearest: 2^-6 at 32 heads; 2^-6 * sqrt(2) and 2^-7 * sqrt(2) at
// 16 and 64 heads, written from the nearest FP32 of sqrt(2) (bits 0x3FB504F3).
float head_weight_scale(int heads) {
    const float sqrt2 = 1.41421353816986083984375f;
    switch (heads) {
        case 16: return sqrt2 * 0.015625f;
        case 32: return 0.015625f;
        default: return sqrt2 * 0.0078125f;
    }
}

hipStream_t as_stream(void *s) { return static_cast<hipStream_t>(s); }

dsaidx_status hip_status(hipError_t e) { return e == hipSuccess ? DSAIDX_OK : DSAIDX_EHIP; }

constexpr int64_t kMaxGrid = 0x7FFFFFFF;
static_assert(dsaidx::kTopkMaxWidth == DSAIDX_TOPK_MAX_WIDTH, "one top-k width limit");
static_assert(dsaidx::kStaticScratchBytes == DSAIDX_STATIC_SCRATCH_BYTES, "one scratch size");

}  // namespace

extern "C" {

const char *dsaidx_status_string(int status) {
    switch (status) {
        case DSAIDX_OK: return "ok";
        case DSAIDX_EINVAL: return "invalid argument";
        case DSAIDX_ELAYOUT: return "unsupported stride, alignment or buffer layout";
        case DSAIDX_EUNSUPPORTED: return "unsupported shape";
        case DSAIDX_EHIP: return "HIP launch error";
        case DSAIDX_ESCRATCH: return "sizes need more than the static scratch of the allocation-free call";
        default: return "unknown status";
    }
}

int64_t dsaidx_query_row_bytes(int fmt, int32_t heads) {
    if (!valid_fmt(fmt) || !valid_heads(heads)) return 0;
    return fmt == DSAIDX_MXFP4 ? (int64_t)heads * 68 : (int64_t)heads * 128;
}

dsaidx_status dsaidx_quantize_queries(int fmt, const void *q, int64_t rows, int32_t heads,
                                      int64_t q_row_stride, int64_t q_head_stride,
                                      const void *wv, int64_t wv_row_stride, void *q_out,
                                      int64_t q_out_row_stride, void *w_out,
                                      int64_t w_out_row_stride, void *stream) {
    if (!valid_fmt(fmt) || rows < 0 || rows > kMaxGrid) return DSAIDX_EINVAL;
    if (!valid_heads(heads)) return DSAIDX_EUNSUPPORTED;
    if (rows == 0) return DSAIDX_OK;
    if (!q || !q_out || (wv && !w_out)) return DSAIDX_EINVAL;
    if (q_head_stride < DSAIDX_DIM || q_row_stride < (int64_t)(heads - 1) * q_head_stride + DSAIDX_DIM)
        return DSAIDX_ELAYOUT;
    if (!aligned(q, 16) || q_head_stride % 8 || q_row_stride % 8) return DSAIDX_ELAYOUT;
    if (!aligned(q_out, 16) || q_out_row_stride % 16 ||
        q_out_row_stride < dsaidx_query_row_bytes(fmt, heads))
        return DSAIDX_ELAYOUT;
    if (wv && (wv_row_stride < heads || w_out_row_stride < heads || !aligned(wv, 2) ||
               !aligned(w_out, 2)))
        return DSAIDX_ELAYOUT;
    return hip_status(dsaidx::launch_quantize_queries(
        fmt, q, rows, heads, q_row_stride, q_head_stride, wv, wv_row_stride, q_out,
        q_out_row_stride, wv ? w_out : nullptr, w_out_row_stride, head_weight_scale(heads),
        as_stream(stream)));
}

dsaidx_status dsaidx_store_keys(int fmt, const void *keys, int64_t tokens, int64_t k_row_stride,
                                const float *gamma, const float *beta, float eps,
                                const int64_t *slots, void *cache, int64_t num_pages,
                                int64_t page_stride, void *stream) {
    if (!valid_fmt(fmt) || tokens < 0 || (tokens + 3) / 4 > kMaxGrid || num_pages < 0)
        return DSAIDX_EINVAL;
    if (!std::isfinite(eps) || eps < 0.0f) return DSAIDX_EINVAL;
    if (tokens == 0) return DSAIDX_OK;
    if (!keys || !gamma || !beta || !slots || !cache) return DSAIDX_EINVAL;
    if (k_row_stride < DSAIDX_DIM || k_row_stride % 2 || !aligned(keys, 4)) return DSAIDX_ELAYOUT;
    if (!aligned(gamma, 8) || !aligned(beta, 8) || !aligned(slots, 8)) return DSAIDX_ELAYOUT;
    if (page_stride < section_bytes(fmt) || page_stride % 16 || !aligned(cache, 16))
        return DSAIDX_ELAYOUT;
    return hip_status(dsaidx::launch_store_keys(fmt, keys, tokens, k_row_stride, gamma, beta, eps,
                                                slots, cache, num_pages, page_stride,
                                                as_stream(stream)));
}

}  // extern "C"

namespace {

// Argument rules of index_inputs; *empty = true when there are no tokens (nothing to launch).
dsaidx_status check_index_inputs(int fmt, const void *projected, int64_t tokens,
                                 int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
                                 const void *q, int32_t heads, int64_t q_row_stride,
                                 int64_t q_head_stride, const float *gamma, const float *beta,
                                 float eps, const int64_t *slots, void *cache, int64_t num_pages,
                                 int64_t page_stride, void *q_out, int64_t q_out_row_stride,
                                 void *w_out, int64_t w_out_row_stride, bool *empty) {
    *empty = false;
    if (!valid_fmt(fmt) || tokens < 0 || tokens > kMaxGrid - 1 || num_pages < 0 || key_col < 0 ||
        weight_col < 0)
        return DSAIDX_EINVAL;
    if (!std::isfinite(eps) || eps < 0.0f) return DSAIDX_EINVAL;
    if (!valid_heads(heads)) return DSAIDX_EUNSUPPORTED;
    if (tokens == 0) {
        *empty = true;
        return DSAIDX_OK;
    }
    if (!projected || !q || !gamma || !beta || !slots || !cache || !q_out || !w_out)
        return DSAIDX_EINVAL;
    // packed row: the key's 128 columns and the H weight columns lie inside each row; the key
    // is read as 4-byte column pairs
    if (proj_row_stride < key_col + DSAIDX_DIM || proj_row_stride < weight_col + heads ||
        !aligned(projected, 4) || proj_row_stride % 2 || key_col % 2)
        return DSAIDX_ELAYOUT;
    if (q_head_stride < DSAIDX_DIM || q_row_stride < (int64_t)(heads - 1) * q_head_stride + DSAIDX_DIM)
        return DSAIDX_ELAYOUT;
    if (!aligned(q, 16) || q_head_stride % 8 || q_row_stride % 8) return DSAIDX_ELAYOUT;
    if (!aligned(q_out, 16) || q_out_row_stride % 16 ||
        q_out_row_stride < dsaidx_query_row_bytes(fmt, heads))
        return DSAIDX_ELAYOUT;
    if (w_out_row_stride < heads || !aligned(w_out, 2)) return DSAIDX_ELAYOUT;
    if (!aligned(gamma, 8) || !aligned(beta, 8) || !aligned(slots, 8)) return DSAIDX_ELAYOUT;
    if (page_stride < section_bytes(fmt) || page_stride % 16 || !aligned(cache, 16))
        return DSAIDX_ELAYOUT;
    return DSAIDX_OK;
}

// Argument rules of decode_layout.
dsaidx_status check_layout(const int32_t *seq_lens, const int32_t *query_lens,
                           int64_t num_requests, int64_t num_rows, int32_t dcp_rank,
                           int32_t dcp_world_size, int32_t interleave, int32_t *query_starts,
                           int32_t *row_ends) {
    if (!(0 <= dcp_rank && dcp_rank < dcp_world_size) || interleave < 1 || num_rows < 0 ||
        num_requests < 0 || num_requests > kMaxGrid || num_rows > kMaxGrid)
        return DSAIDX_EINVAL;
    if (!query_starts || (num_rows > 0 && !row_ends) ||
        (num_requests > 0 && (!seq_lens || !query_lens)))
        return DSAIDX_EINVAL;
    if (!aligned(query_starts, 4) || (row_ends && !aligned(row_ends, 4))) return DSAIDX_ELAYOUT;
    return DSAIDX_OK;
}

}  // namespace

extern "C" {

dsaidx_status dsaidx_index_inputs(int fmt, const void *projected, int64_t tokens,
                                  int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
                                  const void *q, int32_t heads, int64_t q_row_stride,
                                  int64_t q_head_stride, const float *gamma, const float *beta,
                                  float eps, const int64_t *slots, void *cache,
                                  int64_t num_pages, int64_t page_stride, void *q_out,
                                  int64_t q_out_row_stride, void *w_out, int64_t w_out_row_stride,
                                  void *stream) {
    bool empty = false;
    const dsaidx_status st = check_index_inputs(
        fmt, projected, tokens, proj_row_stride, key_col, weight_col, q, heads, q_row_stride,
        q_head_stride, gamma, beta, eps, slots, cache, num_pages, page_stride, q_out,
        q_out_row_stride, w_out, w_out_row_stride, &empty);
    if (st != DSAIDX_OK || empty) return st;
    return hip_status(dsaidx::launch_index_inputs(
        fmt, projected, tokens, proj_row_stride, key_col, weight_col, q, heads, q_row_stride,
        q_head_stride, gamma, beta, eps, slots, cache, num_pages, page_stride, q_out,
        q_out_row_stride, w_out, w_out_row_stride, head_weight_scale(heads), nullptr,
        as_stream(stream)));
}

dsaidx_status dsaidx_index_inputs_layout(
    int fmt, const void *projected, int64_t tokens, int64_t proj_row_stride, int64_t key_col,
    int64_t weight_col, const void *q, int32_t heads, int64_t q_row_stride,
    int64_t q_head_stride, const float *gamma, const float *beta, float eps,
    const int64_t *slots, void *cache, int64_t num_pages, int64_t page_stride, void *q_out,
    int64_t q_out_row_stride, void *w_out, int64_t w_out_row_stride, const int32_t *seq_lens,
    const int32_t *query_lens, int64_t num_requests, int64_t num_rows, int32_t dcp_rank,
    int32_t dcp_world_size, int32_t interleave, int32_t *query_starts, int32_t *row_ends,
    void *stream) {
    bool empty = false;
    dsaidx_status st = check_index_inputs(
        fmt, projected, tokens, proj_row_stride, key_col, weight_col, q, heads, q_row_stride,
        q_head_stride, gamma, beta, eps, slots, cache, num_pages, page_stride, q_out,
        q_out_row_stride, w_out, w_out_row_stride, &empty);
    if (st != DSAIDX_OK) return st;
    st = check_layout(seq_lens, query_lens, num_requests, num_rows, dcp_rank, dcp_world_size,
                      interleave, query_starts, row_ends);
    if (st != DSAIDX_OK) return st;
    const dsaidx::LayoutArgs la{seq_lens, query_lens, num_requests, num_rows, dcp_rank,
                                dcp_world_size, interleave, query_starts, row_ends};
    return hip_status(dsaidx::launch_index_inputs(
        fmt, projected, tokens, proj_row_stride, key_col, weight_col, q, heads, q_row_stride,
        q_head_stride, gamma, beta, eps, slots, cache, num_pages, page_stride, q_out,
        q_out_row_stride, w_out, w_out_row_stride, head_weight_scale(heads), &la,
        as_stream(stream)));
}

dsaidx_status dsaidx_decode_layout(const int32_t *seq_lens, const int32_t *query_lens,
                                   int64_t num_requests, int64_t num_rows, int32_t dcp_rank,
                                   int32_t dcp_world_size, int32_t interleave,
                                   int32_t *query_starts, int32_t *row_ends, void *stream) {
    const dsaidx_status st = check_layout(seq_lens, query_lens, num_requests, num_rows, dcp_rank,
                                          dcp_world_size, interleave, query_starts, row_ends);
    if (st != DSAIDX_OK) return st;
    return hip_status(dsaidx::launch_decode_layout(seq_lens, query_lens, num_requests, num_rows,
                                                   dcp_rank, dcp_world_size, interleave,
                                                   query_starts, row_ends, as_stream(stream)));
}

dsaidx_status dsaidx_score_paged(int fmt, const void *q, int64_t q_row_stride, int32_t heads,
                                 const void *w, int64_t w_row_stride, const void *cache,
                                 int64_t num_pages, int64_t page_stride,
                                 const int32_t *block_table, int64_t num_requests,
                                 int64_t max_blocks, const int32_t *query_starts,
                                 const int32_t *row_ends, int64_t num_rows,
                                 int32_t max_query_len, float *logits,
                                 int64_t logits_row_stride, void *stream) {
    if (!valid_fmt(fmt) || num_rows < 0 || num_requests < 0 || max_blocks < 0 || num_pages < 0)
        return DSAIDX_EINVAL;
    if (!valid_heads(heads) || max_query_len < 1 || max_query_len > DSAIDX_MAX_QUERY_LEN)
        return DSAIDX_EUNSUPPORTED;
    if (num_rows == 0 || num_requests == 0 || max_blocks == 0 || num_pages == 0) return DSAIDX_OK;
    if (!q || !w || !cache || !block_table || !query_starts || !row_ends || !logits)
        return DSAIDX_EINVAL;
    if (!aligned(q, 16) || q_row_stride % 16 || q_row_stride < dsaidx_query_row_bytes(fmt, heads))
        return DSAIDX_ELAYOUT;
    if (!aligned(w, 8) || w_row_stride % 4 || w_row_stride < heads) return DSAIDX_ELAYOUT;
    if (page_stride < section_bytes(fmt) || page_stride % 16 || !aligned(cache, 16))
        return DSAIDX_ELAYOUT;
    if (max_blocks > (int64_t)INT32_MAX / DSAIDX_PAGE_TOKENS ||
        logits_row_stride < max_blocks * DSAIDX_PAGE_TOKENS || !aligned(logits, 4))
        return DSAIDX_ELAYOUT;
    const int64_t chunks = (max_blocks + 7) / 8;  // at least 2 pages per wavefront, 4 wavefronts
    if (chunks * num_requests > kMaxGrid) return DSAIDX_EUNSUPPORTED;
    dsaidx::ScoreArgs a{fmt,         q,          q_row_stride, heads,         w,
                        w_row_stride, cache,     num_pages,    page_stride,   block_table,
                        num_requests, max_blocks, query_starts, row_ends,     num_rows,
                        max_query_len, logits,    logits_row_stride};
    return hip_status(dsaidx::launch_score_paged(a, as_stream(stream)));
}

size_t dsaidx_score_topk_workspace_bytes(int64_t num_requests, int64_t max_blocks,
                                         int64_t num_rows) {
    if (num_requests < 1 || max_blocks < 1 || num_rows < 0 || max_blocks > (int64_t)INT32_MAX / 64)
        return 0;
    if (dsaidx::score_geometry(num_requests, max_blocks).chunks > dsaidx::kMaxRowSegments) return 0;
    return dsaidx::score_topk_workspace_bytes(num_requests, max_blocks, num_rows);
}

int64_t dsaidx_score_segment_keys(int64_t num_requests, int64_t max_blocks) {
    if (num_requests < 1 || max_blocks < 1 || max_blocks > (int64_t)INT32_MAX / 64) return 0;
    return dsaidx::score_geometry(num_requests, max_blocks).segment_keys;
}

int64_t dsaidx_read_sections_words(int64_t num_requests, int64_t max_blocks) {
    if (num_requests < 1 || max_blocks < 1 || max_blocks > (int64_t)INT32_MAX / 64) return 0;
    return dsaidx::read_sections_words(num_requests, max_blocks);
}

dsaidx_status dsaidx_read_sections(int fmt, const void *cache, int64_t num_pages,
                                   int64_t page_stride, const int32_t *block_table,
                                   int64_t num_requests, int64_t max_blocks,
                                   const int32_t *seq_lens, uint32_t *out, int64_t out_words,
                                   void *stream) {
    if (!valid_fmt(fmt) || num_requests < 0 || max_blocks < 0 || num_pages < 0 || out_words < 0)
        return DSAIDX_EINVAL;
    if (num_requests == 0 || max_blocks == 0 || num_pages == 0) return DSAIDX_OK;
    if (!cache || !block_table || !seq_lens || !out) return DSAIDX_EINVAL;
    if (page_stride < section_bytes(fmt) || page_stride % 16 || !aligned(cache, 16) ||
        !aligned(out, 4) || max_blocks > (int64_t)INT32_MAX / DSAIDX_PAGE_TOKENS)
        return DSAIDX_ELAYOUT;
    const int64_t words = dsaidx::read_sections_words(num_requests, max_blocks);
    if (words / dsaidx::kScoreWaves > kMaxGrid) return DSAIDX_EUNSUPPORTED;
    if (out_words < words) return DSAIDX_EINVAL;
    return hip_status(dsaidx::launch_read_sections(fmt, cache, num_pages, page_stride, block_table,
                                                   num_requests, max_blocks, seq_lens, out,
                                                   as_stream(stream)));
}

dsaidx_status dsaidx_read_stream(const void *buf, int64_t bytes, int32_t workgroups,
                                 uint32_t *out, int64_t out_words, void *stream) {
    if (bytes < 0 || bytes % 16 || workgroups < 1 || workgroups > (1 << 20) || out_words < 0)
        return DSAIDX_EINVAL;
    if (bytes == 0) return DSAIDX_OK;
    if (!buf || !out || !aligned(buf, 16) || !aligned(out, 4) || out_words < 4 * (int64_t)workgroups)
        return DSAIDX_EINVAL;
    return hip_status(dsaidx::launch_read_stream(buf, bytes, workgroups, out, as_stream(stream)));
}

dsaidx_status dsaidx_score_paged_hist(int fmt, const void *q, int64_t q_row_stride,
                                      int32_t heads, const void *w, int64_t w_row_stride,
                                      const void *cache, int64_t num_pages, int64_t page_stride,
                                      const int32_t *block_table, int64_t num_requests,
                                      int64_t max_blocks, const int32_t *query_starts,
                                      const int32_t *row_ends, int64_t num_rows,
                                      int32_t max_query_len, float *logits,
                                      int64_t logits_row_stride, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    // the argument rules of score_paged first (a dry run: launch nothing yet)
    if (!valid_fmt(fmt) || num_rows < 0 || num_requests < 0 || max_blocks < 0 || num_pages < 0)
        return DSAIDX_EINVAL;
    if (!valid_heads(heads) || max_query_len < 1 || max_query_len > DSAIDX_MAX_QUERY_LEN)
        return DSAIDX_EUNSUPPORTED;
    if (num_rows == 0 || num_requests == 0 || max_blocks == 0 || num_pages == 0) return DSAIDX_OK;
    if (!q || !w || !cache || !block_table || !query_starts || !row_ends || !logits)
        return DSAIDX_EINVAL;
    if (!aligned(q, 16) || q_row_stride % 16 || q_row_stride < dsaidx_query_row_bytes(fmt, heads))
        return DSAIDX_ELAYOUT;
    if (!aligned(w, 8) || w_row_stride % 4 || w_row_stride < heads) return DSAIDX_ELAYOUT;
    if (page_stride < section_bytes(fmt) || page_stride % 16 || !aligned(cache, 16))
        return DSAIDX_ELAYOUT;
    if (max_blocks > (int64_t)INT32_MAX / DSAIDX_PAGE_TOKENS ||
        logits_row_stride < max_blocks * DSAIDX_PAGE_TOKENS || !aligned(logits, 4))
        return DSAIDX_ELAYOUT;
    const dsaidx::ScoreGeometry geo = dsaidx::score_geometry(num_requests, max_blocks);
    if (geo.chunks * num_requests > kMaxGrid || geo.chunks > dsaidx::kMaxRowSegments)
        return DSAIDX_EUNSUPPORTED;
    const size_t need = dsaidx::score_topk_workspace_bytes(num_requests, max_blocks, num_rows);
    if (!workspace || workspace_bytes < need) return DSAIDX_EINVAL;
    if (!aligned(workspace, 256)) return DSAIDX_ELAYOUT;
    dsaidx::ScoreArgs a{fmt,         q,          q_row_stride, heads,         w,
                        w_row_stride, cache,     num_pages,    page_stride,   block_table,
                        num_requests, max_blocks, query_starts, row_ends,     num_rows,
                        max_query_len, logits,    logits_row_stride};
    return hip_status(dsaidx::launch_score_paged_hist(a, workspace, as_stream(stream)));
}

int64_t dsaidx_decode_tile_size(int64_t max_model_len, int64_t width, int32_t topk,
                                int32_t heads) {
    if (max_model_len < 0 || width < 0 || topk < 1 || heads < 1 ||
        max_model_len > ((int64_t)1 << 40) || width > ((int64_t)1 << 40))
        return 0;
    const int64_t row_bytes = 4 * width + 24 * (topk < width ? (int64_t)topk : width) +
                              64 * (int64_t)heads + 256;
    const int64_t rows = 32 * 4 * max_model_len / (row_bytes > 1 ? row_bytes : 1);
    return rows > 32 ? rows : 32;
}

size_t dsaidx_score_topk_tiled_workspace_bytes(int64_t num_requests, int64_t max_blocks,
                                               int64_t tile_rows, int32_t max_query_len) {
    if (num_requests < 1 || max_blocks < 1 || tile_rows < 1 || max_query_len < 1 ||
        max_query_len > DSAIDX_MAX_QUERY_LEN || max_blocks > (int64_t)INT32_MAX / 64)
        return 0;
    const int64_t gr = dsaidx::tiled_geometry_requests(num_requests, tile_rows, max_query_len);
    if (dsaidx::score_geometry(gr, max_blocks).chunks > dsaidx::kMaxRowSegments) return 0;
    return dsaidx::score_topk_tiled_workspace_bytes(num_requests, max_blocks, tile_rows,
                                                    max_query_len);
}

dsaidx_status dsaidx_score_topk_tiled(int fmt, const void *q, int64_t q_row_stride,
                                      int32_t heads, const void *w, int64_t w_row_stride,
                                      const void *cache, int64_t num_pages, int64_t page_stride,
                                      const int32_t *block_table, int64_t num_requests,
                                      int64_t max_blocks, const int32_t *query_starts,
                                      const int32_t *row_ends, int64_t num_rows,
                                      int32_t max_query_len, int32_t k, int32_t *indices,
                                      int64_t indices_row_stride, int64_t tile_rows,
                                      float *logits_tile, int64_t logits_tile_row_stride,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_fmt(fmt) || num_rows < 0 || num_requests < 0 || max_blocks < 0 || num_pages < 0 ||
        k < 1 || tile_rows < 1)
        return DSAIDX_EINVAL;
    if (!valid_heads(heads) || max_query_len < 1 || max_query_len > DSAIDX_MAX_QUERY_LEN)
        return DSAIDX_EUNSUPPORTED;
    if (num_rows == 0) return DSAIDX_OK;
    if (num_requests == 0 || max_blocks == 0 || num_pages == 0)
        return DSAIDX_EINVAL;  // rows to select for, and no scoring geometry
    if (!q || !w || !cache || !block_table || !query_starts || !row_ends || !logits_tile ||
        !indices || !workspace)
        return DSAIDX_EINVAL;
    if (!aligned(q, 16) || q_row_stride % 16 || q_row_stride < dsaidx_query_row_bytes(fmt, heads))
        return DSAIDX_ELAYOUT;
    if (!aligned(w, 8) || w_row_stride % 4 || w_row_stride < heads) return DSAIDX_ELAYOUT;
    if (page_stride < section_bytes(fmt) || page_stride % 16 || !aligned(cache, 16))
        return DSAIDX_ELAYOUT;
    if (max_blocks > (int64_t)INT32_MAX / DSAIDX_PAGE_TOKENS ||
        logits_tile_row_stride < max_blocks * DSAIDX_PAGE_TOKENS || !aligned(logits_tile, 4) ||
        indices_row_stride < k || !aligned(indices, 4))
        return DSAIDX_ELAYOUT;
    const int64_t gr = dsaidx::tiled_geometry_requests(num_requests, tile_rows, max_query_len);
    const dsaidx::ScoreGeometry geo = dsaidx::score_geometry(gr, max_blocks);
    if (geo.chunks * num_requests > kMaxGrid || geo.chunks > dsaidx::kMaxRowSegments ||
        tile_rows * (geo.chunks + 1) > kMaxGrid)
        return DSAIDX_EUNSUPPORTED;
    if (workspace_bytes < dsaidx::score_topk_tiled_workspace_bytes(num_requests, max_blocks,
                                                                   tile_rows, max_query_len))
        return DSAIDX_EINVAL;
    if (!aligned(workspace, 256)) return DSAIDX_ELAYOUT;
    const dsaidx::ScoreArgs a{fmt,         q,          q_row_stride, heads,         w,
                              w_row_stride, cache,     num_pages,    page_stride,   block_table,
                              num_requests, max_blocks, query_starts, row_ends,     num_rows,
                              max_query_len, logits_tile, logits_tile_row_stride};
    return hip_status(dsaidx::launch_score_topk_tiled(a, k, indices, indices_row_stride, tile_rows,
                                                      workspace, as_stream(stream)));
}

// The checks of the step calls (index_score_hist, index_score_topk) and their launch arguments.
// Returns DSAIDX_OK with `*layout_only` set where nothing is scored (the row layout alone).
static dsaidx_status index_step_args(
    int fmt, const void *projected, int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
    const void *q, int32_t heads, int64_t q_row_stride, int64_t q_head_stride, const float *gamma,
    const float *beta, float eps, const int32_t *seq_lens, const int32_t *query_lens,
    int64_t num_requests, int64_t num_rows, int32_t max_query_len, void *cache, int64_t num_pages,
    int64_t page_stride, const int32_t *block_table, int64_t max_blocks, int32_t *query_starts,
    int32_t *row_ends, float *logits, int64_t logits_row_stride, void *workspace,
    size_t workspace_bytes, bool *layout_only, dsaidx::ScoreArgs *args, dsaidx::FusedInputs *fin) {
    if (!valid_fmt(fmt) || num_rows < 0 || num_requests < 0 || max_blocks < 0 || num_pages < 0 ||
        key_col < 0 || weight_col < 0 || !std::isfinite(eps) || eps < 0.0f)
        return DSAIDX_EINVAL;
    if (!valid_heads(heads) || max_query_len < 1 ||
        max_query_len > dsaidx::index_score_max_query_len(fmt))
        return DSAIDX_EUNSUPPORTED;
    dsaidx_status st = check_layout(seq_lens, query_lens, num_requests, num_rows, 0, 1, 1,
                                    query_starts, row_ends);
    if (st != DSAIDX_OK) return st;
    // nothing to score and no key with a place in the cache: the row layout alone
    *layout_only = num_rows == 0 || num_requests == 0 || max_blocks == 0 || num_pages == 0;
    if (*layout_only) return DSAIDX_OK;
    if (!projected || !q || !gamma || !beta || !cache || !block_table || !logits)
        return DSAIDX_EINVAL;
    // the index-input rules (packed rows, BF16 query rows, LayerNorm parameters)
    if (proj_row_stride < key_col + DSAIDX_DIM || proj_row_stride < weight_col + heads ||
        !aligned(projected, 4) || proj_row_stride % 2 || key_col % 2)
        return DSAIDX_ELAYOUT;
    if (q_head_stride < DSAIDX_DIM || q_row_stride < (int64_t)(heads - 1) * q_head_stride + DSAIDX_DIM)
        return DSAIDX_ELAYOUT;
    if (!aligned(q, 16) || q_head_stride % 8 || q_row_stride % 8) return DSAIDX_ELAYOUT;
    if (!aligned(gamma, 8) || !aligned(beta, 8)) return DSAIDX_ELAYOUT;
    // the scoring rules
    if (page_stride < section_bytes(fmt) || page_stride % 16 || !aligned(cache, 16))
        return DSAIDX_ELAYOUT;
    if (max_blocks > (int64_t)INT32_MAX / DSAIDX_PAGE_TOKENS ||
        logits_row_stride < max_blocks * DSAIDX_PAGE_TOKENS || !aligned(logits, 4))
        return DSAIDX_ELAYOUT;
    const dsaidx::ScoreGeometry geo = dsaidx::score_geometry(num_requests, max_blocks);
    if (geo.chunks * num_requests > kMaxGrid || geo.chunks > dsaidx::kMaxRowSegments)
        return DSAIDX_EUNSUPPORTED;
    const size_t need = dsaidx::score_topk_workspace_bytes(num_requests, max_blocks, num_rows);
    if (!workspace || workspace_bytes < need) return DSAIDX_EINVAL;
    if (!aligned(workspace, 256)) return DSAIDX_ELAYOUT;
    // `q` carries the BF16 query and `query_starts` the query lengths in this mode
    *args = dsaidx::ScoreArgs{fmt,          q,          q_row_stride, heads,      nullptr,
                              0,            cache,      num_pages,    page_stride, block_table,
                              num_requests, max_blocks, query_lens,   nullptr,    num_rows,
                              max_query_len, logits,    logits_row_stride};
    auto *pp = static_cast<const uint16_t *>(projected);
    *fin = dsaidx::FusedInputs{seq_lens, pp + key_col, pp + weight_col, proj_row_stride,
                               q_head_stride, gamma, beta, eps, head_weight_scale(heads),
                               query_starts, row_ends};
    return DSAIDX_OK;
}

dsaidx_status dsaidx_index_score_hist(
    int fmt, const void *projected, int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
    const void *q, int32_t heads, int64_t q_row_stride, int64_t q_head_stride, const float *gamma,
    const float *beta, float eps, const int32_t *seq_lens, const int32_t *query_lens,
    int64_t num_requests, int64_t num_rows, int32_t max_query_len, void *cache, int64_t num_pages,
    int64_t page_stride, const int32_t *block_table, int64_t max_blocks, int32_t *query_starts,
    int32_t *row_ends, float *logits, int64_t logits_row_stride, void *workspace,
    size_t workspace_bytes, void *stream) {
    bool layout_only = false;
    dsaidx::ScoreArgs a{};
    dsaidx::FusedInputs fin{};
    const dsaidx_status st = index_step_args(
        fmt, projected, proj_row_stride, key_col, weight_col, q, heads, q_row_stride,
        q_head_stride, gamma, beta, eps, seq_lens, query_lens, num_requests, num_rows,
        max_query_len, cache, num_pages, page_stride, block_table, max_blocks, query_starts,
        row_ends, logits, logits_row_stride, workspace, workspace_bytes, &layout_only, &a, &fin);
    if (st != DSAIDX_OK) return st;
    if (layout_only)
        return hip_status(dsaidx::launch_decode_layout(seq_lens, query_lens, num_requests,
                                                       num_rows, 0, 1, 1, query_starts,
                                                       row_ends, as_stream(stream)));
    return hip_status(dsaidx::launch_index_score_hist(a, fin, workspace, as_stream(stream)));
}

dsaidx_status dsaidx_index_score_topk(
    int fmt, const void *projected, int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
    const void *q, int32_t heads, int64_t q_row_stride, int64_t q_head_stride, const float *gamma,
    const float *beta, float eps, const int32_t *seq_lens, const int32_t *query_lens,
    int64_t num_requests, int64_t num_rows, int32_t max_query_len, void *cache, int64_t num_pages,
    int64_t page_stride, const int32_t *block_table, int64_t max_blocks, int32_t *query_starts,
    int32_t *row_ends, float *logits, int64_t logits_row_stride, int32_t k, int32_t *indices,
    int64_t indices_row_stride, void *workspace, size_t workspace_bytes, void *stream) {
    if (k < 1) return DSAIDX_EINVAL;
    bool layout_only = false;
    dsaidx::ScoreArgs a{};
    dsaidx::FusedInputs fin{};
    const dsaidx_status st = index_step_args(
        fmt, projected, proj_row_stride, key_col, weight_col, q, heads, q_row_stride,
        q_head_stride, gamma, beta, eps, seq_lens, query_lens, num_requests, num_rows,
        max_query_len, cache, num_pages, page_stride, block_table, max_blocks, query_starts,
        row_ends, logits, logits_row_stride, workspace, workspace_bytes, &layout_only, &a, &fin);
    if (st != DSAIDX_OK) return st;
    if (layout_only)
        return hip_status(dsaidx::launch_decode_layout(seq_lens, query_lens, num_requests,
                                                       num_rows, 0, 1, 1, query_starts,
                                                       row_ends, as_stream(stream)));
    // the selection's rules (as topk_scored)
    if (!indices) return DSAIDX_EINVAL;
    if (indices_row_stride < k || !aligned(indices, 4)) return DSAIDX_ELAYOUT;
    const int64_t chunks = dsaidx::score_geometry(num_requests, max_blocks).chunks;
    if (num_rows * (chunks + 1) > kMaxGrid) return DSAIDX_EUNSUPPORTED;
    a.select_k = k;
    a.select_out = indices;
    a.select_stride = indices_row_stride;
    return hip_status(dsaidx::launch_index_score_topk(a, fin, workspace, as_stream(stream)));
}

dsaidx_status dsaidx_topk_scored(const float *logits, int64_t num_rows, int64_t logits_row_stride,
                                 const int32_t *row_ends, int32_t k, int32_t *indices,
                                 int64_t indices_row_stride, int64_t num_requests,
                                 int64_t max_blocks, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    if (num_rows < 0 || num_requests < 0 || max_blocks < 0 || k < 1) return DSAIDX_EINVAL;
    if (num_rows == 0) return DSAIDX_OK;
    if (num_requests == 0 || max_blocks == 0) return DSAIDX_EINVAL;  // no scoring geometry
    if (!row_ends || !indices || !logits || !workspace) return DSAIDX_EINVAL;
    if (max_blocks > (int64_t)INT32_MAX / DSAIDX_PAGE_TOKENS) return DSAIDX_ELAYOUT;
    const int64_t width = max_blocks * DSAIDX_PAGE_TOKENS;
    if (logits_row_stride < width || indices_row_stride < k || !aligned(logits, 4) ||
        !aligned(indices, 4))
        return DSAIDX_ELAYOUT;
    const dsaidx::ScoreGeometry geo = dsaidx::score_geometry(num_requests, max_blocks);
    if (geo.chunks > dsaidx::kMaxRowSegments || num_rows * (geo.chunks + 1) > kMaxGrid)
        return DSAIDX_EUNSUPPORTED;
    if (workspace_bytes < dsaidx::score_topk_workspace_bytes(num_requests, max_blocks, num_rows))
        return DSAIDX_EINVAL;
    if (!aligned(workspace, 256)) return DSAIDX_ELAYOUT;
    return hip_status(dsaidx::launch_topk_after_histograms(
        logits, num_rows, width, logits_row_stride, row_ends, k, indices, indices_row_stride,
        workspace, geo.chunks, geo.segment_keys, as_stream(stream)));
}

size_t dsaidx_topk_workspace_bytes(int64_t rows, int64_t width, int32_t k) {
    if (rows < 0 || width < 0 || width > DSAIDX_TOPK_MAX_WIDTH || k < 1) return 0;
    return dsaidx::topk_workspace_bytes(rows, width, k);
}

dsaidx_status dsaidx_topk(const float *logits, int64_t rows, int64_t width,
                          int64_t logits_row_stride, const int32_t *row_ends, int32_t k,
                          int32_t *indices, int64_t indices_row_stride, void *workspace,
                          size_t workspace_bytes, void *stream) {
    if (rows < 0 || width < 0 || k < 1) return DSAIDX_EINVAL;
    if (width > DSAIDX_TOPK_MAX_WIDTH || rows * ((width + 4095) / 4096 + 1) > kMaxGrid)
        return DSAIDX_EUNSUPPORTED;
    if (rows == 0) return DSAIDX_OK;
    if (!row_ends || !indices || (width > 0 && !logits)) return DSAIDX_EINVAL;
    if (logits_row_stride < width || indices_row_stride < k || !aligned(logits, 4) ||
        !aligned(indices, 4))
        return DSAIDX_ELAYOUT;
    const size_t need = dsaidx::topk_workspace_bytes(rows, width, k);
    if (workspace_bytes < need || (need > 0 && !workspace)) return DSAIDX_EINVAL;
    if (!aligned(workspace, 256)) return DSAIDX_ELAYOUT;
    return hip_status(dsaidx::launch_topk(logits, rows, width, logits_row_stride, row_ends, k,
                                          indices, indices_row_stride, workspace,
                                          workspace_bytes, as_stream(stream)));
}

dsaidx_status dsaidx_topk_noalloc(const float *logits, int64_t rows, int64_t width,
                                  int64_t logits_row_stride, const int32_t *row_ends, int32_t k,
                                  int32_t *indices, int64_t indices_row_stride, void *stream) {
    if (rows < 0 || width < 0 || k < 1) return DSAIDX_EINVAL;
    if (width > DSAIDX_TOPK_MAX_WIDTH || rows * ((width + 4095) / 4096 + 1) > kMaxGrid)
        return DSAIDX_EUNSUPPORTED;
    if (rows == 0) return DSAIDX_OK;
    if (!row_ends || !indices || (width > 0 && !logits)) return DSAIDX_EINVAL;
    if (logits_row_stride < width || indices_row_stride < k || !aligned(logits, 4) ||
        !aligned(indices, 4))
        return DSAIDX_ELAYOUT;
    if (dsaidx::topk_workspace_bytes(rows, width, k) > dsaidx::kStaticScratchBytes)
        return DSAIDX_ESCRATCH;
    void *ws = nullptr;
    if (dsaidx::static_scratch(&ws) != hipSuccess) return DSAIDX_EHIP;
    return hip_status(dsaidx::launch_topk(logits, rows, width, logits_row_stride, row_ends, k,
                                          indices, indices_row_stride, ws,
                                          dsaidx::kStaticScratchBytes, as_stream(stream)));
}

dsaidx_status dsaidx_dcp_candidates(const float *logits, int64_t rows, int64_t width,
                                    int64_t logits_row_stride, const int32_t *indices, int32_t k,
                                    int64_t indices_row_stride, int32_t dcp_rank,
                                    int32_t dcp_world_size, int32_t interleave, float *values,
                                    int32_t *positions, void *stream) {
    if (rows < 0 || width < 0 || k < 1 || interleave < 1 || dcp_world_size < 1 ||
        !(0 <= dcp_rank && dcp_rank < dcp_world_size))
        return DSAIDX_EINVAL;
    if ((width + interleave) * (int64_t)dcp_world_size > INT32_MAX || rows * ((k + 255) / 256) > kMaxGrid)
        return DSAIDX_EUNSUPPORTED;
    if (rows == 0) return DSAIDX_OK;
    if (!indices || !values || !positions || (width > 0 && !logits)) return DSAIDX_EINVAL;
    if (logits_row_stride < width || indices_row_stride < k || !aligned(logits, 4) ||
        !aligned(indices, 4) || !aligned(values, 4) || !aligned(positions, 4))
        return DSAIDX_ELAYOUT;
    return hip_status(dsaidx::launch_dcp_candidates(logits, rows, width, logits_row_stride,
                                                    indices, k, indices_row_stride, dcp_rank,
                                                    dcp_world_size, interleave, values, positions,
                                                    as_stream(stream)));
}

dsaidx_status dsaidx_dcp_merge(const float *values, const int32_t *positions,
                               int32_t dcp_world_size, int64_t rows, int32_t kc, int32_t k,
                               int32_t *merged, int64_t merged_row_stride, int32_t dcp_rank,
                               int32_t interleave, int32_t *local_slots,
                               int64_t local_row_stride, void *stream) {
    if (rows < 0 || kc < 1 || k < 1 || dcp_world_size < 1 || interleave < 1 || rows > kMaxGrid)
        return DSAIDX_EINVAL;
    if (local_slots && !(0 <= dcp_rank && dcp_rank < dcp_world_size)) return DSAIDX_EINVAL;
    if ((int64_t)dcp_world_size * kc > dsaidx::kDcpMergeCap) return DSAIDX_EUNSUPPORTED;
    if (rows == 0) return DSAIDX_OK;
    if (!values || !positions || !merged) return DSAIDX_EINVAL;
    if (merged_row_stride < k || (local_slots && local_row_stride < k) || !aligned(values, 4) ||
        !aligned(positions, 4) || !aligned(merged, 4) || !aligned(local_slots, 4))
        return DSAIDX_ELAYOUT;
    return hip_status(dsaidx::launch_dcp_merge(values, positions, dcp_world_size, rows, kc, k,
                                               merged, merged_row_stride, dcp_rank, interleave,
                                               local_slots, local_row_stride, as_stream(stream)));
}

}  // extern "C"
