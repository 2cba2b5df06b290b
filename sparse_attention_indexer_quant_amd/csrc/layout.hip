// Row bounds of grouped verify rows, on the device (no device-to-host reads).
//
// Page "vllm.models.kimi_k3.amd.ops.fp4_indexer", decode_layout: query_starts =
// [0, cumsum(query_lens)]; a row's request is the count of query_starts[1..R] <= row,
// clamped to the last request; its key bound is max(0, seq - qlen + row - start + 1);
// under decode context parallelism the bound becomes the rank's share of keys dealt out
// in runs of `interleave`; rows at or past query_starts[R] are graph padding with bound 0.
#include "device_common.h"
#include "launch.h"

namespace dsaidx {

constexpr int kLayoutThreads = 1024;

// Inclusive prefix sum over the workgroup (16 wavefronts); `partials` holds 16 ints.
__device__ __forceinline__ int block_scan_1024(int v, int *partials) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int n = __shfl_up(v, d);
        if (lane >= d) v += n;
    }
    if (lane == 63) partials[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int s = lane < 16 ? partials[lane] : 0;
#pragma unroll
        for (int d = 1; d < 16; d <<= 1) {
            const int n = __shfl_up(s, d);
            if (lane >= d) s += n;
        }
        if (lane < 16) partials[lane] = s;
    }
    __syncthreads();
    if (wave > 0) v += partials[wave - 1];
    __syncthreads();
    return v;
}

__global__ __launch_bounds__(kLayoutThreads) void decode_layout_kernel(
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ query_lens, int64_t R,
    int64_t num_rows, int dcp_rank, int dcp_world, int interleave, int32_t *__restrict__ starts,
    int32_t *__restrict__ row_ends) {
    __shared__ int partials[16];
    __shared__ int carry;
    const int tid = threadIdx.x;
    if (tid == 0) {
        starts[0] = 0;
        carry = 0;
    }
    __syncthreads();
    for (int64_t base = 0; base < R; base += kLayoutThreads) {
        const int64_t i = base + tid;
        const int v = i < R ? query_lens[i] : 0;
        const int incl = block_scan_1024(v, partials);
        const int c = carry;
        if (i < R) starts[i + 1] = c + incl;
        __syncthreads();
        if (tid == kLayoutThreads - 1) carry = c + incl;
        __syncthreads();
    }
    const int64_t total = carry;  // query_starts[R]
    __threadfence_block();
    __syncthreads();
    for (int64_t row = tid; row < num_rows; row += kLayoutThreads) {
        if (R == 0 || row >= total) {
            row_ends[row] = 0;
            continue;
        }
        // first request index j with starts[j + 1] > row
        int64_t lo = 0, hi = R;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (starts[mid + 1] <= row) lo = mid + 1;
            else hi = mid;
        }
        const int64_t req = lo < R - 1 ? lo : R - 1;
        int64_t end = (int64_t)seq_lens[req] - query_lens[req] + row - starts[req] + 1;
        if (end < 0) end = 0;
        if (dcp_world > 1) {
            const int64_t il = interleave;
            const int64_t full = end / (dcp_world * il) * il;
            int64_t local = end - full * dcp_world - (int64_t)dcp_rank * il;
            local = local < 0 ? 0 : (local > il ? il : local);
            end = full + local;
        }
        row_ends[row] = (int32_t)end;
    }
}

hipError_t launch_decode_layout(const int32_t *seq_lens, const int32_t *query_lens,
                                int64_t num_requests, int64_t num_rows, int dcp_rank,
                                int dcp_world_size, int interleave, int32_t *query_starts,
                                int32_t *row_ends, hipStream_t stream) {
    hipLaunchKernelGGL(decode_layout_kernel, dim3(1), dim3(kLayoutThreads), 0, stream, seq_lens,
                       query_lens, num_requests, num_rows, dcp_rank, dcp_world_size, interleave,
                       query_starts, row_ends);
    return hipGetLastError();
}

}  // namespace dsaidx
