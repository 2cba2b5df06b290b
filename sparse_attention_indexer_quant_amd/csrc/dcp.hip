// Decode context parallelism (DCP) around the top-k on gfx950.
//
// Page "vllm.models.kimi_k3.amd.ops.fp4_indexer", decode_layout: under DCP the keys of a
// request are dealt to the ranks in runs of `interleave` (run j to rank j % W as that rank's
// run j / W), and each rank scores only its own keys against rank-local row bounds. Page
// "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.overlap", module text: the
// indexer path then ends in a top-k merge and the local slots.
//
//   dcp_candidates: one rank's local top-k as (logit, global position) pairs, the payload an
//     all-gather over the ranks would carry (8 B per candidate).
//   dcp_merge: per row, the k largest of all ranks' candidates, ties to the lower global
//     position (-0 equals +0), as global positions; optionally also the rank-local positions
//     of the selected keys that one rank owns (its local slots). Each rank's local top-k
//     holds every one of its keys that can be in the global top-k (local order of a rank's
//     keys is their global order), so the merge is the global top-k of the whole row.
//
// The merge keeps all W * k candidates of a row in LDS as 63-bit composites
// (inverted order key << 31 | global position), unique per key, and radix-selects the k
// smallest.
#include "device_common.h"
#include "launch.h"
#include "select.h"

namespace dsaidx {

constexpr int kMergeCap = kDcpMergeCap;  // candidates per row kept in LDS (128 KB)

__device__ __forceinline__ int64_t dcp_global(int64_t local, int rank, int world, int interleave) {
    return (local / interleave) * ((int64_t)world * interleave) + (int64_t)rank * interleave +
           local % interleave;
}

__global__ __launch_bounds__(256) void dcp_candidates_kernel(
    const float *__restrict__ logits, int64_t width, int64_t logits_row_stride,
    const int32_t *__restrict__ indices, int k, int64_t indices_row_stride, int rank, int world,
    int interleave, float *__restrict__ values, int32_t *__restrict__ positions,
    int64_t chunks_per_row) {
    const int64_t row = blockIdx.x / chunks_per_row;
    const int64_t j = (blockIdx.x % chunks_per_row) * 256 + threadIdx.x;
    if (j >= k) return;
    const int32_t idx = indices[row * indices_row_stride + j];
    const bool ok = idx >= 0 && idx < width;
    values[row * k + j] = ok ? logits[row * logits_row_stride + idx] : -INFINITY;
    positions[row * k + j] = ok ? (int32_t)dcp_global(idx, rank, world, interleave) : -1;
}

struct MergeShared {
    uint64_t cand[kMergeCap];
    SelectShared<> sel;
    uint32_t n_valid;
    uint32_t n_local;
};

__global__ __launch_bounds__(kSelectThreads) void dcp_merge_kernel(
    const float *__restrict__ values, const int32_t *__restrict__ positions, int world,
    int64_t rows, int kc, int k, int32_t *__restrict__ merged, int64_t merged_row_stride,
    int rank, int interleave, int32_t *__restrict__ local_slots, int64_t local_row_stride) {
    __shared__ MergeShared sh;
    const int64_t row = blockIdx.x;
    if (threadIdx.x == 0) {
        sh.n_valid = 0;
        sh.n_local = 0;
    }
    __syncthreads();
    // gather the row's valid candidates from every rank's slice [world][rows][kc]
    const int total = world * kc;
    for (int i = threadIdx.x; i < total; i += kSelectThreads) {
        const int w = i / kc, j = i % kc;
        const int64_t at = ((int64_t)w * rows + row) * kc + j;
        const int32_t g = positions[at];
        if (g < 0) continue;
        const uint64_t c = ((uint64_t)(~order_key(values[at])) << 31) | (uint32_t)g;
        sh.cand[atomicAdd(&sh.n_valid, 1u)] = c;
    }
    __syncthreads();
    const int m = (int)sh.n_valid;
    const int take = m < k ? m : k;
    int32_t *out = merged + row * merged_row_stride;
    int32_t *loc = local_slots ? local_slots + row * local_row_stride : nullptr;
    if (take > 0) {
        const uint64_t t = select_threshold(LdsCandidates<>{sh.cand, m}, take, 63, sh.sel);
        if (threadIdx.x == 0) sh.sel.n_out = 0;
        __syncthreads();
        for (int i = threadIdx.x; i < m; i += kSelectThreads) {
            const uint64_t c = sh.cand[i];
            if (c > t) continue;
            const int32_t g = (int32_t)(c & 0x7FFFFFFFu);
            const uint32_t slot = atomicAdd(&sh.sel.n_out, 1u);
            if (slot < (uint32_t)take) out[slot] = g;
            if (loc && (g / interleave) % world == rank) {
                const uint32_t ls = atomicAdd(&sh.n_local, 1u);
                if (ls < (uint32_t)k) loc[ls] = (g / ((int64_t)interleave * world)) * interleave + g % interleave;
            }
        }
        __syncthreads();
    }
    for (int i = take + threadIdx.x; i < k; i += kSelectThreads) out[i] = -1;
    if (loc)
        for (int i = (int)sh.n_local + threadIdx.x; i < k; i += kSelectThreads) loc[i] = -1;
}

hipError_t launch_dcp_candidates(const float *logits, int64_t rows, int64_t width,
                                 int64_t logits_row_stride, const int32_t *indices, int k,
                                 int64_t indices_row_stride, int rank, int world, int interleave,
                                 float *values, int32_t *positions, hipStream_t stream) {
    const int64_t chunks = (k + 255) / 256;
    hipLaunchKernelGGL(dcp_candidates_kernel, dim3((unsigned)(rows * chunks)), dim3(256), 0,
                       stream, logits, width, logits_row_stride, indices, k, indices_row_stride,
                       rank, world, interleave, values, positions, chunks);
    return hipGetLastError();
}

hipError_t launch_dcp_merge(const float *values, const int32_t *positions, int world,
                            int64_t rows, int kc, int k, int32_t *merged,
                            int64_t merged_row_stride, int rank, int interleave,
                            int32_t *local_slots, int64_t local_row_stride, hipStream_t stream) {
    hipLaunchKernelGGL(dcp_merge_kernel, dim3((unsigned)rows), dim3(kSelectThreads), 0, stream,
                       values, positions, world, rows, kc, k, merged, merged_row_stride, rank,
                       interleave, local_slots, local_row_stride);
    return hipGetLastError();
}

}  // namespace dsaidx
