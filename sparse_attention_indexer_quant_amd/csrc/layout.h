// Row bounds of grouped verify rows, on the device (no device-to-host reads): the body that
// one workgroup runs, shared by the decode_layout kernel and the fused step-input kernel.
//
// Page "vllm.models.kimi_k3.amd.ops.fp4_indexer", decode_layout: query_starts =
// [0, cumsum(query_lens)]; a row's request is the count of query_starts[1..R] <= row,
// clamped to the last request; its key bound is max(0, seq - qlen + row - start + 1);
// under decode context parallelism the bound becomes the rank's share of keys dealt out
// in runs of `interleave`; rows at or past query_starts[R] are graph padding with bound 0.
#pragma once

#include "device_common.h"
#include "select.h"

namespace dsaidx {

struct LayoutArgs {
    const int32_t *seq_lens;
    const int32_t *query_lens;
    int64_t num_requests;
    int64_t num_rows;
    int dcp_rank, dcp_world, interleave;
    int32_t *starts;
    int32_t *row_ends;
};

// Run by all NT lanes of one workgroup. Lane i of each block of NT requests scans the query
// lengths and then writes its own request's rows (query lengths are small: decode and verify
// rows); the rows past the last request are padding. Each request's length and sequence
// length are loaded together, so the whole layout costs one round trip per NT requests.
template <int NT>
__device__ __forceinline__ void decode_layout_body(const LayoutArgs &a) {
    __shared__ int partials[NT / 64];
    __shared__ int carry;
    const int tid = threadIdx.x;
    const int64_t R = a.num_requests;
    if (tid == 0) {
        a.starts[0] = 0;
        carry = 0;
    }
    __syncthreads();
    for (int64_t base = 0; base < R; base += NT) {
        const int64_t i = base + tid;
        const int v = i < R ? a.query_lens[i] : 0;
        const int seq = i < R ? a.seq_lens[i] : 0;
        const int incl = scan_block<NT>(v, partials);
        const int c = carry;
        if (i < R) {
            a.starts[i + 1] = c + incl;
            const int64_t start = (int64_t)c + incl - v;
            // row start + r of this request: end = max(0, seq - qlen + r + 1)
            for (int r = 0; r < v && start + r < a.num_rows; ++r) {
                int64_t end = (int64_t)seq - v + r + 1;
                if (end < 0) end = 0;
                if (a.dcp_world > 1) {
                    const int64_t il = a.interleave;
                    const int64_t full = end / (a.dcp_world * il) * il;
                    int64_t local = end - full * a.dcp_world - (int64_t)a.dcp_rank * il;
                    local = local < 0 ? 0 : (local > il ? il : local);
                    end = full + local;
                }
                a.row_ends[start + r] = (int32_t)end;
            }
        }
        __syncthreads();
        if (tid == NT - 1) carry = c + incl;
        __syncthreads();
    }
    const int64_t total = carry;  // query_starts[R]: rows from here on are graph padding
    for (int64_t row = (total > 0 ? total : 0) + tid; row < a.num_rows; row += NT)
        a.row_ends[row] = 0;
}

}  // namespace dsaidx
