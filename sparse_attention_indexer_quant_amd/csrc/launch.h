// Host-side launchers of the gfx950 kernels. The C-ABI layer (capi.cpp) validates every
// argument first and only then calls these; each returns the HIP error of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

constexpr int64_t kTopkMaxWidth = int64_t(1) << 25;  // keys per row that topk accepts

hipError_t launch_quantize_queries(int fmt, const void *q, int64_t rows, int heads,
                                   int64_t q_row_stride, int64_t q_head_stride, const void *wv,
                                   int64_t wv_row_stride, void *q_out, int64_t q_out_row_stride,
                                   void *w_out, int64_t w_out_row_stride, float c_h,
                                   hipStream_t stream);

hipError_t launch_store_keys(int fmt, const void *keys, int64_t tokens, int64_t k_row_stride,
                             const float *gamma, const float *beta, float eps,
                             const int64_t *slots, void *cache, int64_t num_pages,
                             int64_t page_stride, hipStream_t stream);

struct LayoutArgs;
// `layout` (may be null): also compute decode_layout in the same launch (one more workgroup).
hipError_t launch_index_inputs(int fmt, const void *projected, int64_t tokens,
                               int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
                               const void *q, int heads, int64_t q_row_stride,
                               int64_t q_head_stride, const float *gamma, const float *beta,
                               float eps, const int64_t *slots, void *cache, int64_t num_pages,
                               int64_t page_stride, void *q_out, int64_t q_out_row_stride,
                               void *w_out, int64_t w_out_row_stride, float c_h,
                               const LayoutArgs *layout, hipStream_t stream);

hipError_t launch_decode_layout(const int32_t *seq_lens, const int32_t *query_lens,
                                int64_t num_requests, int64_t num_rows, int dcp_rank,
                                int dcp_world_size, int interleave, int32_t *query_starts,
                                int32_t *row_ends, hipStream_t stream);

struct ScoreArgs {
    int fmt;
    const void *q;
    int64_t q_row_stride;
    int heads;
    const void *w;
    int64_t w_row_stride;
    const void *cache;
    int64_t num_pages;
    int64_t page_stride;
    const int32_t *block_table;
    int64_t num_requests;
    int64_t max_blocks;
    const int32_t *query_starts;
    const int32_t *row_ends;
    int64_t num_rows;
    int max_query_len;
    float *logits;
    int64_t logits_row_stride;
    // the row window [row_lo, num_rows): logits and histograms of row r at row r - row_lo
    int64_t row_lo = 0;
    // requests the launch geometry is sized for (0: num_requests)
    int64_t geometry_requests = 0;
    // the selection made by the scoring launch itself (launch_index_score_topk, rows of one
    // scoring workgroup each): k, and the [num_rows, >= k] positions with their row stride
    int select_k = 0;
    int32_t *select_out = nullptr;
    int64_t select_stride = 0;
};

hipError_t launch_score_paged(const ScoreArgs &args, hipStream_t stream);

// The step's inputs, made inside the scorer (index_score_hist, MXFP4): in ScoreArgs, `q` is
// then the BF16 query [rows, H, 128] (q_row_stride in elements), `query_starts` the query
// lengths, and `w` / `row_ends` are unused.
struct FusedInputs {
    const int32_t *seq_lens;
    const uint16_t *key_in;  // key column of projection row 0 (BF16)
    const uint16_t *w_in;    // head-weight column of projection row 0 (BF16)
    int64_t proj_row_stride;
    int64_t q_head_stride;
    const float *gamma, *beta;
    float eps, c_h;
    int32_t *query_starts;   // written: [0, cumsum(query_lens)]
    int32_t *row_ends;       // written: decode_layout's row bounds
};

hipError_t launch_index_score_hist(const ScoreArgs &args, const FusedInputs &fin,
                                   void *workspace, hipStream_t stream);
// The most rows per request index_score_hist takes for a format (4 MXFP4, 2 FP8).
int index_score_max_query_len(int fmt);
// index_score_hist and the selection of every row's top-k (a.select_k, a.select_out,
// a.select_stride): one launch where each request has one row and every row's keys lie in one
// scoring workgroup (the workgroup selects from its own histogram and logits), else
// index_score_hist followed by the selection on its histograms (topk_scored).
hipError_t launch_index_score_topk(const ScoreArgs &args, const FusedInputs &fin,
                                   void *workspace, hipStream_t stream);

// How score_paged splits a request's pages: pages per wavefront, workgroups ("chunks") per
// request, and the keys one workgroup covers (the top-k segment when the scorer writes the
// selection's histograms). Depends on the current device's compute-unit count.
constexpr int kScoreWaves = 4;  // wavefronts per scoring workgroup
// Compute units of the current device (queried once per device).
int device_cus();
struct ScoreGeometry {
    int pages_per_wave;
    int64_t chunks;
    int64_t segment_keys;
};
ScoreGeometry score_geometry(int64_t num_requests, int64_t max_blocks);

// Scoring that also writes the top-k segment histograms into a top-k workspace laid out for
// (num_rows, chunks) segments; then launch_topk_after_histograms finishes the selection.
size_t score_topk_workspace_bytes(int64_t num_requests, int64_t max_blocks, int64_t num_rows);
hipError_t launch_score_paged_hist(const ScoreArgs &a, void *workspace, hipStream_t stream);

// Row-tiled scoring + selection ([fp4ops] decode_tile_size): the logits buffer and the
// workspace hold one tile of `tile_rows` rows; indices are written for every row.
int64_t tiled_geometry_requests(int64_t num_requests, int64_t tile_rows, int max_query_len);
size_t score_topk_tiled_workspace_bytes(int64_t num_requests, int64_t max_blocks, int64_t tile_rows,
                                        int max_query_len);
hipError_t launch_score_topk_tiled(const ScoreArgs &a, int k, int32_t *indices,
                                   int64_t indices_row_stride, int64_t tile_rows,
                                   void *workspace, hipStream_t stream);

// Decode context parallelism: one rank's merge candidates, and the merge.
constexpr int kDcpMergeCap = 16384;  // world * candidates per rank, per row
hipError_t launch_dcp_candidates(const float *logits, int64_t rows, int64_t width,
                                 int64_t logits_row_stride, const int32_t *indices, int k,
                                 int64_t indices_row_stride, int rank, int world, int interleave,
                                 float *values, int32_t *positions, hipStream_t stream);
hipError_t launch_dcp_merge(const float *values, const int32_t *positions, int world,
                            int64_t rows, int kc, int k, int32_t *merged,
                            int64_t merged_row_stride, int rank, int interleave,
                            int32_t *local_slots, int64_t local_row_stride, hipStream_t stream);

// A plain read of the sections score_paged reads, in its grid (a bandwidth reference): one
// The allocation-free top-k's device scratch: its size, the devices it serves, and its
// address on the current device (taken on the first call there, kept after).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxScratchDevices = 64;
hipError_t static_scratch(void **out);

// A contiguous read of `bytes` (a multiple of 16) by `workgroups` workgroups of 256 lanes,
// one XOR word per wavefront into `out` (4 * workgroups words).
hipError_t launch_read_stream(const void *buf, int64_t bytes, int workgroups, uint32_t *out,
                              hipStream_t stream);
// XOR word per wavefront into `out` (read_sections_words words).
int64_t read_sections_words(int64_t num_requests, int64_t max_blocks);
hipError_t launch_read_sections(int fmt, const void *cache, int64_t num_pages, int64_t page_stride,
                                const int32_t *block_table, int64_t num_requests,
                                int64_t max_blocks, const int32_t *seq_lens, uint32_t *out,
                                hipStream_t stream);

size_t topk_workspace_bytes(int64_t rows, int64_t width, int k);
hipError_t launch_topk_after_histograms(const float *logits, int64_t rows, int64_t width,
                                        int64_t logits_row_stride, const int32_t *row_ends, int k,
                                        int32_t *indices, int64_t indices_row_stride,
                                        void *workspace, int64_t nseg, int64_t seg_len,
                                        hipStream_t stream);

hipError_t launch_topk(const float *logits, int64_t rows, int64_t width, int64_t logits_row_stride,
                       const int32_t *row_ends, int k, int32_t *indices,
                       int64_t indices_row_stride, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

}  // namespace dsaidx
