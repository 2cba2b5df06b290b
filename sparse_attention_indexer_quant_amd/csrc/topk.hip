// Per-row top-k of the indexer scores on gfx950.
//
// Page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.overlap", module text:
// the indexer path is scoring and then top-k. The selection returns the k largest logits
// of [0, row_end) with ties going to the lower key position (-0 counts as +0); fewer than
// k keys give all of them and -1 after. The order within a row is not specified.
//
// One workgroup (16 wavefronts) per row. Logits map to order-preserving 32-bit keys; three
// LDS histogram passes over 11 + 11 + 10 key bits pin the exact k-th largest key T and how
// many keys equal to T belong to the set. A final pass in index order writes every key
// above T and the lowest-indexed keys equal to T, with positions from a workgroup prefix
// sum, so the result set is deterministic.
#include "device_common.h"
#include "launch.h"

namespace dsaidx {

constexpr int kTopkThreads = 1024;

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0;  // -0 == +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int topk_block_scan(int v, int *partials) {
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

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(
    const float *__restrict__ logits, int64_t width, int64_t logits_row_stride,
    const int32_t *__restrict__ row_ends, int k, int32_t *__restrict__ indices,
    int64_t indices_row_stride) {
    __shared__ uint32_t hist[2048];
    __shared__ int partials[16];
    __shared__ uint32_t sel_bin;
    __shared__ int sel_above;
    __shared__ int chunk_total;
    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x;
    int64_t n = row_ends[row];
    n = n < 0 ? 0 : (n > width ? width : n);
    int32_t *out = indices + row * indices_row_stride;
    if (n <= k) {
        for (int i = tid; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        return;
    }
    const float *x = logits + row * logits_row_stride;

    uint32_t prefix = 0, mask = 0;
    int remaining = k;  // how many of the selected keys still lie in the current bin range
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nb = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < 2048; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int64_t i = tid; i < n; i += kTopkThreads) {
            const uint32_t u = order_key(x[i]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        // Thread t owns bins nb-1-t*bpt down to nb-bpt*(t+1) (descending key order).
        const int bpt = nb / kTopkThreads;
        int own = 0;
        for (int j = 0; j < bpt; ++j) own += hist[nb - 1 - (tid * bpt + j)];
        const int incl = topk_block_scan(own, partials);
        int before = incl - own;
        for (int j = 0; j < bpt; ++j) {
            const int bin = nb - 1 - (tid * bpt + j);
            const int c = hist[bin];
            if (before < remaining && before + c >= remaining) {
                sel_bin = (uint32_t)bin;
                sel_above = before;
            }
            before += c;
        }
        __syncthreads();
        prefix |= sel_bin << shift;
        mask |= (uint32_t)(nb - 1) << shift;
        remaining -= sel_above;
        __syncthreads();
    }
    // prefix is now the k-th largest key T; (k - remaining) keys are above it and the
    // `remaining` lowest-indexed keys equal to T complete the set.
    const uint32_t T = prefix;
    const int count_gt = k - remaining;
    int gt_base = 0, eq_base = 0;
#pragma unroll 1
    for (int64_t base = 0; base < n; base += 4 * kTopkThreads) {
        uint32_t u[4];
        int g = 0, e = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = base + tid * 4 + j;
            u[j] = i < n ? order_key(x[i]) : 0u;
            g += i < n && u[j] > T;
            e += i < n && u[j] == T;
        }
        const int mine = g | (e << 16);
        const int incl = topk_block_scan(mine, partials);
        const int excl = incl - mine;
        int gpos = gt_base + (excl & 0xFFFF);
        int epos = eq_base + (excl >> 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t i = base + tid * 4 + j;
            if (i >= n) break;
            if (u[j] > T) {
                out[gpos++] = (int32_t)i;
            } else if (u[j] == T) {
                if (epos < remaining) out[count_gt + epos] = (int32_t)i;
                ++epos;
            }
        }
        if (tid == kTopkThreads - 1) chunk_total = incl;
        __syncthreads();
        gt_base += chunk_total & 0xFFFF;
        eq_base += chunk_total >> 16;
        __syncthreads();
    }
}

size_t topk_workspace_bytes(int64_t, int64_t, int) { return 0; }

hipError_t launch_topk(const float *logits, int64_t rows, int64_t width, int64_t logits_row_stride,
                       const int32_t *row_ends, int k, int32_t *indices,
                       int64_t indices_row_stride, void *, size_t, hipStream_t stream) {
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)rows), dim3(kTopkThreads), 0, stream, logits,
                       width, logits_row_stride, row_ends, k, indices, indices_row_stride);
    return hipGetLastError();
}

}  // namespace dsaidx
