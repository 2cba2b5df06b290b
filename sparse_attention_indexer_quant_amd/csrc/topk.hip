// Per-row top-k of the indexer scores on gfx950.
//
// Page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.overlap", module text:
// the indexer path is scoring and then top-k. The selection returns the k largest logits
// of [0, row_end) with ties going to the lower key position (-0 counts as +0); fewer than
// k keys give all of them and -1 after. The order within a row is not specified.
//
// Logits map to order-preserving 32-bit keys u. Four kernels, which communicate only
// through the workspace across kernel boundaries (handing work to a last-arriving workgroup
// needs a device-scope fence per workgroup, an L2 write-back on every XCD, and atomics on a
// row's shared counters serialize; both measured slower than the selection itself):
//
//   1. topk_hist (rows x segments): each workgroup histograms the top 12 key bits of its
//      segment in LDS and stores the counts (16-bit) in the workspace. (The scorer can write
//      these histograms itself, segment = one scoring workgroup's keys; then the selection
//      starts at step 2.)
//   2. topk_threshold (one workgroup per row): rows with row_end <= k are written here
//      directly. Otherwise it sums the row's segment histograms, finds the bin b holding the
//      k-th largest key, then counts each segment's keys above b and inside b and stores
//      their exclusive prefix sums over the segments: every segment's first output slot and
//      first candidate slot.
//   3. topk_collect (rows x segments): writes the positions of keys above bin b to the
//      output and the (key, position) pairs of keys inside bin b to the row's candidate
//      list, at the offsets from step 2 plus an in-workgroup prefix sum -- no atomics, and
//      the positions above b come out in ascending order.
//   4. topk_select (one workgroup per row): loads the candidates into LDS as the composite
//      (low 20 key bits inverted, position), unique per key, and radix-selects the
//      `remaining` smallest, so exactly the keys with the largest values -- ties to the
//      lower position -- are taken. A bin that overflowed the candidate list is selected
//      from the row itself instead.
//
// Standalone segments are 4096 keys, doubled (up to 32768) until rows x segments is at most
// 2048 workgroups and a row has at most 1024 segments (rows hold at most 2^25 keys). Every
// workspace field is written before it is read within a call, so the workspace needs no
// initialisation; calls sharing one must be ordered.
#include "device_common.h"
#include "launch.h"
#include "select.h"
#include "topk_layout.h"

namespace dsaidx {

constexpr int kTopkThreads = 256;
constexpr int kRowThreads = 1024;        // threshold: one workgroup per row
constexpr int kMinSegment = 4096;        // keys per workgroup (doubled for many rows)
constexpr int kMaxSegment = 32768;       // 16-bit segment histogram counts stay exact
constexpr int kMaxWorkgroups = 2048;
static_assert(kTopkMaxWidth / kMaxSegment <= kMaxRowSegments, "a row fits the threshold kernel");
static_assert(kMaxRowSegments <= kRowThreads, "one thread per segment in the offset scan");

// Keys per segment for this call's shape (the same rule sizes the workspace).
inline int64_t topk_segment(int64_t rows, int64_t width) {
    int64_t seg = kMinSegment;
    while (seg < kMaxSegment && (rows * ((width + seg - 1) / seg) > kMaxWorkgroups ||
                                 (width + seg - 1) / seg > kMaxRowSegments))
        seg *= 2;
    return seg;
}

inline int64_t topk_nseg(int64_t width, int64_t seg) { return width > 0 ? (width + seg - 1) / seg : 1; }

__device__ __forceinline__ int64_t row_bound(const int32_t *row_ends, int64_t row, int64_t width) {
    int64_t n = row_ends[row];
    return n < 0 ? 0 : (n > width ? width : n);
}

template <int VEC, typename F>
__device__ __forceinline__ void for_segment(const float *x, int64_t lo, int64_t hi, F &&fn) {
    if constexpr (VEC == 4) {
        const int64_t hi4 = lo + ((hi - lo) & ~(int64_t)3);
        for (int64_t i = lo + 4 * threadIdx.x; i < hi4; i += 4 * kTopkThreads) {
            const float4 v = *reinterpret_cast<const float4 *>(x + i);
            fn(i, v.x);
            fn(i + 1, v.y);
            fn(i + 2, v.z);
            fn(i + 3, v.w);
        }
        for (int64_t i = hi4 + threadIdx.x; i < hi; i += kTopkThreads) fn(i, x[i]);
    } else {
        for (int64_t i = lo + threadIdx.x; i < hi; i += kTopkThreads) fn(i, x[i]);
    }
}

template <int VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(
    const float *__restrict__ logits, int64_t width, int64_t logits_row_stride,
    const int32_t *__restrict__ row_ends, int k, TopkWorkspace ws, int64_t nseg,
    int64_t seg_len) {
    __shared__ __align__(16) uint32_t hist[kBins];
    const int64_t row = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t n = row_bound(row_ends, row, width);
    if (n <= k) return;   // written by the threshold kernel
    const int64_t lo = seg * seg_len;
    if (lo >= n) return;  // only the segments that hold keys take part below
    const int64_t hi = lo + seg_len < n ? lo + seg_len : n;
    const float *x = logits + row * logits_row_stride;

    for (int b = threadIdx.x; b < kBins; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for_segment<VEC>(x, lo, hi, [&](int64_t, float v) {
        atomicAdd(&hist[order_key(v) >> kBinShift], 1u);
    });
    __syncthreads();
    // lane t stores bins [16t, 16t+16) as 16-bit counts
    uint32_t c[8];
    const uint4 *h4 = reinterpret_cast<const uint4 *>(hist) + 4 * threadIdx.x;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint4 q = h4[v];
        c[2 * v] = q.x | (q.y << 16);
        c[2 * v + 1] = q.z | (q.w << 16);
    }
    uint4 *dst = reinterpret_cast<uint4 *>(ws.seghist + (row * nseg + seg) * kBins +
                                           16 * threadIdx.x);
    dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
    dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
}

// One workgroup per row: a row with at most k keys is written whole (all positions, then
// -1); otherwise the threshold bin and every segment's output offsets.
__global__ __launch_bounds__(kRowThreads) void topk_threshold_kernel(
    const int32_t *__restrict__ row_ends, int64_t width, int k, int32_t *__restrict__ indices,
    int64_t indices_row_stride, TopkWorkspace ws, int64_t nseg, int64_t seg_len) {
    __shared__ __align__(16) uint32_t part_hist[kRowThreads / 256][kBins];  // per segment group
    __shared__ uint32_t seg_above[kMaxRowSegments];
    __shared__ int partials[kRowThreads / 64];
    __shared__ uint32_t found_bin, found_count, top_bin;
    __shared__ int found_above;
    const int64_t row = blockIdx.x;
    const int64_t n = row_bound(row_ends, row, width);
    if (n <= k) {
        int32_t *out = indices + row * indices_row_stride;
        for (int i = threadIdx.x; i < k; i += kRowThreads) out[i] = i < n ? i : -1;
        return;
    }
    const int row_segments = (int)((n + seg_len - 1) / seg_len);
    const uint16_t *rowhist = ws.seghist + row * nseg * kBins;
    const int t = threadIdx.x;

    // (a) Thread t sums bins [16 (t % 256), +16) over the segments s = t / 256 (mod 4),
    // four segments' loads in flight at a time, and stores the sums for its segment group
    // (plain vector stores: every entry is written, nothing to clear, no atomics).
    if (t == 0) {
        found_bin = kBins;  // kept only if the counts do not reach k (they always do)
        found_above = k;
        found_count = 0;
        top_bin = 0;
    }
    {
        const int blk = t & 255, sg0 = t >> 8;
        uint32_t sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};  // bin pairs, 16 bits each
        uint32_t hi16[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        int s = sg0;
        for (; s + 12 < row_segments; s += 16) {
            uint4 v[4][2];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint4 *src = reinterpret_cast<const uint4 *>(rowhist + (int64_t)(s + 4 * u) * kBins + 16 * blk);
                v[u][0] = src[0];
                v[u][1] = src[1];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t w[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w,
                                       v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    sum[e] += w[e] & 0xFFFFu;
                    hi16[e] += w[e] >> 16;
                }
            }
        }
        for (; s < row_segments; s += 4) {
            const uint4 *src = reinterpret_cast<const uint4 *>(rowhist + (int64_t)s * kBins + 16 * blk);
            const uint4 a = src[0], b = src[1];
            const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sum[e] += w[e] & 0xFFFFu;
                hi16[e] += w[e] >> 16;
            }
        }
        uint4 *dst = reinterpret_cast<uint4 *>(&part_hist[sg0][16 * blk]);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            dst[v] = make_uint4(sum[2 * v], hi16[2 * v], sum[2 * v + 1], hi16[2 * v + 1]);
    }
    __syncthreads();

    // (b) Thread t owns bins 4095 - 4t - j, j < 4 (descending): the bin holding the k-th
    // largest key, the keys above it, and the highest non-empty bin (the one where the
    // descending count first leaves zero; a single thread sees that).
    uint4 m4 = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int g = 0; g < kRowThreads / 256; ++g) {
        const uint4 v = reinterpret_cast<const uint4 *>(part_hist[g])[kBins / 4 - 1 - t];
        m4.x += v.x;
        m4.y += v.y;
        m4.z += v.z;
        m4.w += v.w;
    }
    const uint32_t mine[4] = {m4.w, m4.z, m4.y, m4.x};
    const int own = (int)(m4.x + m4.y + m4.z + m4.w);
    const int incl = scan_block<kRowThreads>(own, partials);
    int before = incl - own;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = (int)mine[j];
        if (before == 0 && c > 0) top_bin = (uint32_t)(kBins - 1 - 4 * t - j);
        if (before < k && before + c >= k) {
            found_bin = (uint32_t)(kBins - 1 - 4 * t - j);
            found_above = before;
            found_count = (uint32_t)c;
        }
        before += c;
    }
    for (int sgi = t; sgi < row_segments; sgi += kRowThreads) seg_above[sgi] = 0;
    __syncthreads();
    const uint32_t bin = found_bin, top = top_bin;

    // (c) Per-segment keys above the bin: the bins (bin, top] of every segment, spread
    // over all threads, summed into LDS per segment.
    if (bin < (uint32_t)kBins && top > bin) {
        const int span = (int)(top - bin);
        const int64_t total = (int64_t)row_segments * span;
        for (int64_t idx = t; idx < total; idx += kRowThreads) {
            const int sgi = (int)(idx / span);
            const int b = (int)(bin + 1 + idx % span);
            const uint32_t c = rowhist[(int64_t)sgi * kBins + b];
            if (c) atomicAdd(&seg_above[sgi], c);
        }
    }
    __syncthreads();

    // (d) Exclusive prefix sums over the segments (one per thread): output and candidate
    // offsets of every segment.
    const uint32_t my_above = t < row_segments ? seg_above[t] : 0u;
    const uint32_t my_in =
        t < row_segments && bin < (uint32_t)kBins ? (uint32_t)rowhist[(int64_t)t * kBins + bin] : 0u;
    const int ia = scan_block<kRowThreads>((int)my_above, partials);
    const int ic = scan_block<kRowThreads>((int)my_in, partials);
    if (t < row_segments)
        ws.segoff[row * nseg + t] = make_uint2((uint32_t)ia - my_above, (uint32_t)ic - my_in);
    if (t == 0) {
        RowState &st = ws.state[row];
        st.bin = bin;
        st.above = found_above;
        st.remaining = k - found_above;
        st.n_cand = found_count;
    }
}

template <int VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_collect_kernel(
    const float *__restrict__ logits, int64_t width, int64_t logits_row_stride,
    const int32_t *__restrict__ row_ends, int k, int32_t *__restrict__ indices,
    int64_t indices_row_stride, TopkWorkspace ws, int64_t nseg, int64_t seg_len) {
    __shared__ int partials[kTopkThreads / 64];
    const int64_t row = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t n = row_bound(row_ends, row, width);
    if (n <= k) return;
    const int64_t lo = seg * seg_len;
    if (lo >= n) return;
    const int64_t hi = lo + seg_len < n ? lo + seg_len : n;
    const float *x = logits + row * logits_row_stride;
    int32_t *out = indices + row * indices_row_stride;
    const RowState &st = ws.state[row];
    const uint32_t bin = st.bin, above = (uint32_t)st.above;
    const uint2 off = ws.segoff[row * nseg + seg];
    uint2 *cand = ws.cand + row * kCandCap;

    // Chunks of 4096 keys (16 per lane, in registers): lane counts and a workgroup prefix
    // sum place every key after the segment's offsets and the earlier chunks' keys.
    constexpr int kPer = 16, kChunk = kPer * kTopkThreads;
    uint32_t base_above = off.x, base_in = off.y;
    for (int64_t cbase = lo; cbase < hi; cbase += kChunk) {
        uint32_t u[kPer];
        const int64_t first = cbase + (int64_t)threadIdx.x * kPer;
        if (VEC == 4 && first + kPer <= hi) {
#pragma unroll
            for (int j = 0; j < kPer; j += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(x + first + j);
                u[j] = order_key(v.x);
                u[j + 1] = order_key(v.y);
                u[j + 2] = order_key(v.z);
                u[j + 3] = order_key(v.w);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j) u[j] = first + j < hi ? order_key(x[first + j]) : 0u;
        }
        int n_above = 0, n_in = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const uint32_t d = u[j] >> kBinShift;
            n_above += first + j < hi && d > bin;
            n_in += first + j < hi && d == bin;
        }
        const int mine = n_above | (n_in << 16);
        const int incl = scan_block<kTopkThreads>(mine, partials);
        uint32_t pa = base_above + ((incl - mine) & 0xFFFF);
        uint32_t pc = base_in + ((incl - mine) >> 16);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = first + j;
            const uint32_t d = u[j] >> kBinShift;
            const bool live = i < hi;
            if (live && d > bin) {
                if (pa < above) out[pa] = (int32_t)i;
                ++pa;
            } else if (live && d == bin) {
                if (pc < (uint32_t)kCandCap) cand[pc] = make_uint2(u[j], (uint32_t)i);
                ++pc;
            }
        }
        // the chunk's totals are the sum of the wave totals the scan left in `partials`
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kTopkThreads / 64; ++w) tot += partials[w];
        base_above += (uint32_t)(tot & 0xFFFF);
        base_in += (uint32_t)(tot >> 16);
        __syncthreads();
    }
}

// Composite of a key inside the threshold bin: smaller for a larger value, and for equal
// values smaller for the lower position; unique per position.
__device__ __forceinline__ uint64_t composite(uint32_t u, uint32_t pos, int pos_bits) {
    return ((uint64_t)(~u & 0xFFFFFu) << pos_bits) | pos;
}

struct RowBin {  // every key of the row inside the threshold bin, read from the logits
    const float *x;
    int64_t n;
    uint32_t bin;
    int pos_bits;
    template <typename F>
    __device__ __forceinline__ void for_each(F &&f) const {
        for (int64_t i = threadIdx.x; i < n; i += kSelectThreads) {
            const uint32_t u = order_key(x[i]);
            if ((u >> kBinShift) == bin) f(composite(u, (uint32_t)i, pos_bits));
        }
    }
};

__global__ __launch_bounds__(kSelectThreads) void topk_select_kernel(
    const float *__restrict__ logits, int64_t width, int64_t logits_row_stride,
    const int32_t *__restrict__ row_ends, int k, int32_t *__restrict__ indices,
    int64_t indices_row_stride, TopkWorkspace ws) {
    __shared__ uint64_t cands[kCandCap];
    __shared__ SelectShared sh;
    const int64_t row = blockIdx.x;
    const int64_t n = row_bound(row_ends, row, width);
    if (n <= k) return;
    const float *x = logits + row * logits_row_stride;
    const RowState &st = ws.state[row];
    const uint32_t bin = st.bin, ncand = st.n_cand;
    const int remaining = st.remaining;
    if (remaining <= 0 || remaining > k) return;
    int32_t *out = indices + row * indices_row_stride + st.above;
    int pos_bits = 1;
    while (pos_bits < 31 && ((int64_t)1 << pos_bits) < n) ++pos_bits;
    const int bits = 20 + pos_bits;
    if (ncand <= (uint32_t)kCandCap) {
        const uint2 *cand = ws.cand + row * kCandCap;
        for (int j = threadIdx.x; j < (int)ncand; j += kSelectThreads) {
            const uint2 e = cand[j];
            cands[j] = composite(e.x, e.y, pos_bits);
        }
        __syncthreads();
        select_smallest(LdsCandidates{cands, (int)ncand}, remaining, bits, pos_bits, out, sh);
    } else {
        select_smallest(RowBin{x, n, bin, pos_bits}, remaining, bits, pos_bits, out, sh);
    }
}

size_t topk_workspace_bytes(int64_t rows, int64_t width, int) {
    return topk_layout_bytes(rows, topk_nseg(width, topk_segment(rows, width)));
}

// Steps 2-4 of the selection, on segment histograms already in the workspace.
hipError_t launch_topk_after_histograms(const float *logits, int64_t rows, int64_t width,
                                        int64_t logits_row_stride, const int32_t *row_ends, int k,
                                        int32_t *indices, int64_t indices_row_stride,
                                        void *workspace, int64_t nseg, int64_t seg_len,
                                        hipStream_t stream) {
    const TopkWorkspace ws = carve(workspace, rows, nseg);
    const dim3 grid((unsigned)(nseg * rows)), block(kTopkThreads);
    const bool vec = (reinterpret_cast<uintptr_t>(logits) & 15) == 0 && logits_row_stride % 4 == 0;
    hipLaunchKernelGGL(topk_threshold_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream,
                       row_ends, width, k, indices, indices_row_stride, ws, nseg, seg_len);
    if (vec)
        hipLaunchKernelGGL(topk_collect_kernel<4>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, indices, indices_row_stride, ws, nseg,
                           seg_len);
    else
        hipLaunchKernelGGL(topk_collect_kernel<1>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, indices, indices_row_stride, ws, nseg,
                           seg_len);
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)rows), dim3(kSelectThreads), 0, stream,
                       logits, width, logits_row_stride, row_ends, k, indices, indices_row_stride,
                       ws);
    return hipGetLastError();
}

hipError_t launch_topk(const float *logits, int64_t rows, int64_t width, int64_t logits_row_stride,
                       const int32_t *row_ends, int k, int32_t *indices,
                       int64_t indices_row_stride, void *workspace, size_t, hipStream_t stream) {
    const int64_t seg_len = topk_segment(rows, width);
    const int64_t nseg = topk_nseg(width, seg_len);
    const TopkWorkspace ws = carve(workspace, rows, nseg);
    const dim3 grid((unsigned)(nseg * rows)), block(kTopkThreads);
    const bool vec = (reinterpret_cast<uintptr_t>(logits) & 15) == 0 && logits_row_stride % 4 == 0;
    if (vec)
        hipLaunchKernelGGL(topk_hist_kernel<4>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, ws, nseg, seg_len);
    else
        hipLaunchKernelGGL(topk_hist_kernel<1>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, ws, nseg, seg_len);
    return launch_topk_after_histograms(logits, rows, width, logits_row_stride, row_ends, k,
                                        indices, indices_row_stride, workspace, nseg, seg_len,
                                        stream);
}

}  // namespace dsaidx
