// Per-row top-k of the indexer scores on gfx950.
//
// Page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.overlap", module text:
// the indexer path is scoring and then top-k. The selection returns the k largest logits
// of [0, row_end) with ties going to the lower key position (-0 counts as +0); fewer than
// k keys give all of them and -1 after. The order within a row is not specified.
//
// Logits map to order-preserving 32-bit keys u. Many workgroups share each row:
//
//   1. topk_hist: every workgroup histograms the top 12 bits of its segment of the row in
//      LDS and stores it (16-bit counts) in the workspace. The last workgroup of the row to
//      finish (an arrival counter) sums the row's segment histograms, finds the bin b that
//      holds the k-th largest key and records how many keys lie above it. (Merging with
//      global atomics instead costs one L2 atomic per non-zero bin per segment, which
//      measured slower than the whole selection.)
//   2. topk_collect: every workgroup writes the positions of its keys above bin b straight
//      into the output (one atomic per 4096 keys) and appends the positions of keys inside
//      bin b to the row's candidate list. The last workgroup to finish selects the missing
//      `remaining` keys among the candidates: a radix select over the composite
//      (low 20 key bits inverted, position), smallest first, which is unique per key, so
//      exactly the keys with the largest values -- ties to the lower position -- are taken.
//      If the bin overflows the candidate list it selects from the row itself instead.
//
// Segments are 4096 keys, doubled (up to 32768) until rows x segments is at most 2048
// workgroups. Rows with row_end <= k are written directly. The workspace's counters are
// zero when a call starts and each call returns them to zero (histograms, candidate lists
// and the per-row threshold fields are rewritten before every use).
#include "device_common.h"
#include "launch.h"

namespace dsaidx {

constexpr int kTopkThreads = 256;
constexpr int kMinSegment = 4096;        // keys per workgroup (doubled for many rows)
constexpr int kMaxSegment = 32768;       // 16-bit segment histogram counts stay exact
constexpr int kMaxWorkgroups = 2048;
constexpr int kBins = 4096;              // top 12 key bits
constexpr int kBinShift = 20;
constexpr int kCandCap = 8192;           // candidate positions kept per row
constexpr int kSelectThreads = 256;

struct RowState {
    uint32_t bin;          // threshold bin
    int32_t above;         // keys above the threshold bin
    int32_t remaining;     // keys still to take from inside the bin
    uint32_t arrive_hist;
    uint32_t arrive_collect;
    uint32_t n_above;      // positions written so far (collect)
    uint32_t n_cand;       // candidates appended so far (collect)
    uint32_t pad;
};

struct TopkWorkspace {
    RowState *state;
    uint16_t *seghist;  // [rows][nseg][kBins]
    int32_t *cand;      // [rows][kCandCap]
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Keys per segment for this call's shape (the same rule sizes the workspace).
inline int64_t topk_segment(int64_t rows, int64_t width) {
    int64_t seg = kMinSegment;
    while (seg < kMaxSegment && rows * ((width + seg - 1) / seg) > kMaxWorkgroups) seg *= 2;
    return seg;
}

inline int64_t topk_nseg(int64_t width, int64_t seg) { return width > 0 ? (width + seg - 1) / seg : 1; }

__host__ __device__ inline TopkWorkspace carve(void *ws, int64_t rows, int64_t nseg) {
    char *p = static_cast<char *>(ws);
    TopkWorkspace w;
    w.state = reinterpret_cast<RowState *>(p);
    p += align256(sizeof(RowState) * rows);
    w.seghist = reinterpret_cast<uint16_t *>(p);
    p += align256(sizeof(uint16_t) * kBins * nseg * rows);
    w.cand = reinterpret_cast<int32_t *>(p);
    return w;
}

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0;  // -0 == +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t load_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive prefix sum over a 256-lane workgroup; `partials` holds 4 ints.
__device__ __forceinline__ int scan256(int v, int *partials) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int n = __shfl_up(v, d);
        if (lane >= d) v += n;
    }
    if (lane == 63) partials[wave] = v;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) before += w < wave ? partials[w] : 0;
    __syncthreads();
    return v + before;
}

__device__ __forceinline__ int64_t row_bound(const int32_t *row_ends, int64_t row, int64_t width) {
    int64_t n = row_ends[row];
    return n < 0 ? 0 : (n > width ? width : n);
}

// Rows with at most k keys: all positions, then -1. Segment s writes [s*seg_len, ...) of
// the k outputs; the last segment also writes whatever lies past the row width.
__device__ __forceinline__ void write_short_row(int32_t *out, int64_t n, int k, int64_t seg,
                                                int64_t nseg, int64_t seg_len) {
    const int64_t lo = seg * seg_len;
    const int64_t hi = seg == nseg - 1 ? (int64_t)k : (lo + seg_len < k ? lo + seg_len : k);
    for (int64_t i = lo + threadIdx.x; i < hi; i += kTopkThreads) out[i] = i < n ? (int32_t)i : -1;
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
    const int32_t *__restrict__ row_ends, int k, int32_t *__restrict__ indices,
    int64_t indices_row_stride, TopkWorkspace ws, int64_t nseg, int64_t seg_len) {
    __shared__ uint32_t hist[kBins];
    __shared__ int partials[4];
    __shared__ int last;
    const int64_t row = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t n = row_bound(row_ends, row, width);
    if (n <= k) {
        write_short_row(indices + row * indices_row_stride, n, k, seg, nseg, seg_len);
        return;
    }
    const int64_t lo = seg * seg_len;
    if (lo >= n) return;  // only the segments that hold keys take part below
    const int64_t hi = lo + seg_len < n ? lo + seg_len : n;
    const uint32_t row_segments = (uint32_t)((n + seg_len - 1) / seg_len);
    const float *x = logits + row * logits_row_stride;

    for (int b = threadIdx.x; b < kBins; b += kTopkThreads) hist[b] = 0;
    __syncthreads();
    for_segment<VEC>(x, lo, hi, [&](int64_t, float v) {
        atomicAdd(&hist[order_key(v) >> kBinShift], 1u);
    });
    __syncthreads();
    // store this segment's histogram: lane t writes bins [16t, 16t+16) as 16-bit counts
    uint16_t *rowhist = ws.seghist + row * nseg * kBins;
    {
        uint32_t c[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            c[j] = hist[16 * threadIdx.x + 2 * j] | (hist[16 * threadIdx.x + 2 * j + 1] << 16);
        uint4 *dst = reinterpret_cast<uint4 *>(rowhist + seg * kBins + 16 * threadIdx.x);
        dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
        dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    }
    __threadfence();
    __syncthreads();
    RowState &st = ws.state[row];
    if (threadIdx.x == 0) last = atomicAdd(&st.arrive_hist, 1u) == row_segments - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();

    // Last workgroup of the row: sum the segment histograms and find the bin holding the
    // k-th largest key. Lane t owns the 16 bins of block 255 - t, walked from the top down.
    constexpr int per = kBins / kTopkThreads;
    static_assert(per == 16, "16 bins per lane");
    uint32_t mine[per];
#pragma unroll
    for (int j = 0; j < per; ++j) mine[j] = 0;
    const int block = kTopkThreads - 1 - threadIdx.x;
    for (uint32_t sgi = 0; sgi < row_segments; ++sgi) {
        const uint4 *src = reinterpret_cast<const uint4 *>(rowhist + sgi * kBins + 16 * block);
        const uint4 lo4 = src[0], hi4 = src[1];
        const uint32_t w[8] = {lo4.x, lo4.y, lo4.z, lo4.w, hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) mine[15 - e] += (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    }
    int own = 0;
#pragma unroll
    for (int j = 0; j < per; ++j) own += (int)mine[j];
    const int incl = scan256(own, partials);
    int before = incl - own;
#pragma unroll
    for (int j = 0; j < per; ++j) {
        const int c = (int)mine[j];
        if (before < k && before + c >= k) {
            st.bin = (uint32_t)(kBins - 1 - (threadIdx.x * per + j));
            st.above = before;
            st.remaining = k - before;
        }
        before += c;
    }
    if (threadIdx.x == 0) {
        st.arrive_hist = 0;
        st.arrive_collect = 0;
        st.n_above = 0;
        st.n_cand = 0;
    }
}

// Radix select of the `r` smallest composites c(i) = (~u(i) & 0xFFFFF) << pos_bits | i over
// a source of positions (i < 2^pos_bits), then writes them to out[0..r). `bits` =
// 20 + pos_bits significant composite bits.
template <typename Source>
__device__ void select_smallest(const Source &src, int r, int bits, int32_t *out,
                                uint32_t *hist, int *partials, uint64_t *sel_prefix,
                                int *sel_below, uint32_t *n_out) {
    uint64_t prefix = 0;
    int done_bits = 0;  // high composite bits already fixed in `prefix`
    const int top = bits;
    while (done_bits < top) {
        const int digit = top - done_bits >= 11 ? 11 : top - done_bits;
        const int shift = top - done_bits - digit;
        const int nb = 1 << digit;
        for (int b = threadIdx.x; b < 2048; b += kSelectThreads) hist[b] = 0;
        __syncthreads();
        src.for_each([&](uint64_t c) {
            if ((c >> (shift + digit)) == (prefix >> (shift + digit)))
                atomicAdd(&hist[(c >> shift) & (uint64_t)(nb - 1)], 1u);
        });
        __syncthreads();
        // ascending: lane t owns bins 8t .. 8t+7
        constexpr int per = 2048 / kSelectThreads;
        int own = 0;
        uint32_t mine[per];
#pragma unroll
        for (int j = 0; j < per; ++j) {
            const int b = threadIdx.x * per + j;
            mine[j] = b < nb ? hist[b] : 0u;
            own += (int)mine[j];
        }
        const int incl = scan256(own, partials);
        int before = incl - own;
#pragma unroll
        for (int j = 0; j < per; ++j) {
            const int c = (int)mine[j];
            if (before < r && before + c >= r) {
                *sel_prefix = prefix | ((uint64_t)(threadIdx.x * per + j) << shift);
                *sel_below = before;
            }
            before += c;
        }
        __syncthreads();
        prefix = *sel_prefix;
        r -= *sel_below;
        done_bits += digit;
        __syncthreads();
    }
    // `prefix` is the r0-th smallest composite; composites are unique, so exactly r0 of them
    // are <= prefix.
    if (threadIdx.x == 0) *n_out = 0;
    __syncthreads();
    const uint64_t T = prefix;
    src.for_each_pos([&](uint64_t c, int64_t pos) {
        if (c <= T) out[atomicAdd(n_out, 1u)] = (int32_t)pos;
    });
}

struct CandidateSource {
    const float *x;
    const int32_t *cand;
    int m;
    int pos_bits;
    template <typename F>
    __device__ void for_each(F &&f) const {
        for (int j = threadIdx.x; j < m; j += kSelectThreads) {
            const int32_t i = cand[j];
            f(((uint64_t)(~order_key(x[i]) & 0xFFFFFu) << pos_bits) | (uint32_t)i);
        }
    }
    template <typename F>
    __device__ void for_each_pos(F &&f) const {
        for (int j = threadIdx.x; j < m; j += kSelectThreads) {
            const int32_t i = cand[j];
            f(((uint64_t)(~order_key(x[i]) & 0xFFFFFu) << pos_bits) | (uint32_t)i, (int64_t)i);
        }
    }
};

struct RowBinSource {  // every key of the row inside the threshold bin
    const float *x;
    int64_t n;
    uint32_t bin;
    int pos_bits;
    template <typename F>
    __device__ void for_each(F &&f) const {
        for (int64_t i = threadIdx.x; i < n; i += kSelectThreads) {
            const uint32_t u = order_key(x[i]);
            if ((u >> kBinShift) == bin) f(((uint64_t)(~u & 0xFFFFFu) << pos_bits) | (uint32_t)i);
        }
    }
    template <typename F>
    __device__ void for_each_pos(F &&f) const {
        for (int64_t i = threadIdx.x; i < n; i += kSelectThreads) {
            const uint32_t u = order_key(x[i]);
            if ((u >> kBinShift) == bin) f(((uint64_t)(~u & 0xFFFFFu) << pos_bits) | (uint32_t)i, i);
        }
    }
};

template <int VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_collect_kernel(
    const float *__restrict__ logits, int64_t width, int64_t logits_row_stride,
    const int32_t *__restrict__ row_ends, int k, int32_t *__restrict__ indices,
    int64_t indices_row_stride, TopkWorkspace ws, int64_t nseg, int64_t seg_len) {
    __shared__ uint32_t hist[2048];
    __shared__ int partials[4];
    __shared__ int last;
    __shared__ uint64_t sel_prefix;
    __shared__ int sel_below;
    __shared__ uint32_t n_out;
    __shared__ uint32_t chunk_base[2];
    const int64_t row = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t n = row_bound(row_ends, row, width);
    if (n <= k) return;
    const int64_t lo = seg * seg_len;
    if (lo >= n) return;
    const int64_t hi = lo + seg_len < n ? lo + seg_len : n;
    const uint32_t row_segments = (uint32_t)((n + seg_len - 1) / seg_len);
    const float *x = logits + row * logits_row_stride;
    int32_t *out = indices + row * indices_row_stride;
    RowState &st = ws.state[row];
    const uint32_t bin = st.bin;
    int32_t *cand = ws.cand + row * kCandCap;

    // Chunks of 4096 keys (16 per lane, in registers): lane counts, a workgroup prefix sum,
    // and one atomic per counter per chunk reserve the output and candidate slots. (Atomics
    // per wavefront on the row's two shared counters serialize in L2.)
    constexpr int kPer = 16, kChunk = kPer * kTopkThreads;
    for (int64_t cbase = lo; cbase < hi; cbase += kChunk) {
        uint32_t d[kPer];
        int n_above = 0, n_in = 0;
        const int64_t first = cbase + (int64_t)threadIdx.x * kPer;
        if (VEC == 4 && first + kPer <= hi) {
#pragma unroll
            for (int j = 0; j < kPer; j += 4) {
                const float4 v = *reinterpret_cast<const float4 *>(x + first + j);
                d[j] = order_key(v.x) >> kBinShift;
                d[j + 1] = order_key(v.y) >> kBinShift;
                d[j + 2] = order_key(v.z) >> kBinShift;
                d[j + 3] = order_key(v.w) >> kBinShift;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPer; ++j) d[j] = first + j < hi ? order_key(x[first + j]) >> kBinShift : 0u;
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            n_above += first + j < hi && d[j] > bin;
            n_in += first + j < hi && d[j] == bin;
        }
        const int mine = n_above | (n_in << 16);
        const int incl = scan256(mine, partials);
        if (threadIdx.x == kTopkThreads - 1) {
            const int tot_above = incl & 0xFFFF, tot_in = incl >> 16;
            chunk_base[0] = tot_above ? atomicAdd(&st.n_above, (uint32_t)tot_above) : 0u;
            chunk_base[1] = tot_in ? atomicAdd(&st.n_cand, (uint32_t)tot_in) : 0u;
        }
        __syncthreads();
        uint32_t pa = chunk_base[0] + ((incl - mine) & 0xFFFF);
        uint32_t pc = chunk_base[1] + ((incl - mine) >> 16);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = cbase + (int64_t)threadIdx.x * kPer + j;
            if (i >= hi) break;
            if (d[j] > bin) {
                out[pa++] = (int32_t)i;
            } else if (d[j] == bin) {
                if (pc < (uint32_t)kCandCap) cand[pc] = (int32_t)i;
                ++pc;
            }
        }
        __syncthreads();
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last = atomicAdd(&st.arrive_collect, 1u) == row_segments - 1;
    __syncthreads();
    if (!last) return;
    __threadfence();

    const int above = st.above, remaining = st.remaining;
    const uint32_t ncand = load_relaxed(&st.n_cand);
    int pos_bits = 1;
    while (pos_bits < 31 && ((int64_t)1 << pos_bits) < n) ++pos_bits;
    const int bits = 20 + pos_bits;
    if (ncand <= (uint32_t)kCandCap) {
        CandidateSource src{x, cand, (int)ncand, pos_bits};
        select_smallest(src, remaining, bits, out + above, hist, partials, &sel_prefix,
                        &sel_below, &n_out);
    } else {
        RowBinSource src{x, n, bin, pos_bits};
        select_smallest(src, remaining, bits, out + above, hist, partials, &sel_prefix,
                        &sel_below, &n_out);
    }
    if (threadIdx.x == 0) {
        st.arrive_collect = 0;
        st.n_above = 0;
        st.n_cand = 0;
    }
}

size_t topk_workspace_bytes(int64_t rows, int64_t width, int) {
    const int64_t nseg = topk_nseg(width, topk_segment(rows, width));
    return align256(sizeof(RowState) * rows) + align256(sizeof(uint16_t) * kBins * nseg * rows) +
           align256(sizeof(int32_t) * (size_t)kCandCap * rows);
}

hipError_t launch_topk(const float *logits, int64_t rows, int64_t width, int64_t logits_row_stride,
                       const int32_t *row_ends, int k, int32_t *indices,
                       int64_t indices_row_stride, void *workspace, size_t, hipStream_t stream) {
    const int64_t seg_len = topk_segment(rows, width);
    const int64_t nseg = topk_nseg(width, seg_len);
    const TopkWorkspace ws = carve(workspace, rows, nseg);
    const dim3 grid((unsigned)(nseg * rows)), block(kTopkThreads);
    const bool vec = (reinterpret_cast<uintptr_t>(logits) & 15) == 0 && logits_row_stride % 4 == 0;
    if (vec) {
        hipLaunchKernelGGL(topk_hist_kernel<4>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, indices, indices_row_stride, ws, nseg, seg_len);
        hipLaunchKernelGGL(topk_collect_kernel<4>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, indices, indices_row_stride, ws, nseg, seg_len);
    } else {
        hipLaunchKernelGGL(topk_hist_kernel<1>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, indices, indices_row_stride, ws, nseg, seg_len);
        hipLaunchKernelGGL(topk_collect_kernel<1>, grid, block, 0, stream, logits, width,
                           logits_row_stride, row_ends, k, indices, indices_row_stride, ws, nseg, seg_len);
    }
    return hipGetLastError();
}

}  // namespace dsaidx
