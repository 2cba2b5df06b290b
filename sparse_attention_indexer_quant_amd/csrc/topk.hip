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
//   1. topk_hist (segments x rows): each workgroup histograms the top 12 key bits of its
//      segment in LDS and stores the counts (16-bit) in the workspace. (The scorer can write
//      these histograms itself, segment = one scoring workgroup's keys; then the selection
//      starts at step 2. It writes a segment's block of 64 fine counts only where the block's
//      coarse sum is nonzero, so the steps below read fine blocks through the coarse sums,
//      fine_word.)
//   2. topk_threshold (one workgroup per row): rows with row_end <= k are written here
//      directly. Otherwise it sums the row's segment histograms, finds the bin b holding the
//      k-th largest key, then counts each segment's keys above b and inside b and stores
//      their exclusive prefix sums over the segments: every segment's first output slot and
//      first candidate slot.
//   3. topk_collect (segments x rows): writes the positions of keys above bin b to the
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
#include <mutex>

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
static_assert(4 * kSelectThreads <= kCandCap, "speculative candidate loads stay in the list");

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

// Row and segment of this workgroup in a grid of nseg x rows workgroups: workgroup b takes
// segment s = b / rows of row (b + s) mod rows (fewer than 2^31 workgroups: 32-bit arithmetic,
// made explicitly uniform so the row arithmetic stays scalar). Workgroups go to the 8 XCDs in
// turn by index, b mod 8; rotating the rows by one per segment makes the segments of one row
// visit the XCDs in turn, so rows of different lengths still give every XCD an equal share.
struct RowSeg {
    int64_t row, seg;
};
__device__ __forceinline__ RowSeg row_segment(int64_t rows) {
    const uint32_t R = (uint32_t)rows;
    const uint32_t sg = __builtin_amdgcn_readfirstlane(blockIdx.x / R);
    uint32_t r = blockIdx.x - sg * R + sg % R;
    if (r >= R) r -= R;
    return {(int64_t)r, (int64_t)sg};
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

// Kernel arguments: the ones the first loads need lead (the library preloads the leading
// arguments into scalar registers at wave launch); the rest are loaded in one batch.
template <int VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(
    const float *__restrict__ logits, int64_t logits_row_stride, int64_t width, int64_t seg_len,
    int64_t rows, const int32_t *__restrict__ row_ends, int k, int64_t nseg,
    uint16_t *__restrict__ seghist, uint16_t *__restrict__ coarse) {
    __shared__ __align__(16) uint32_t hist[kBins];
    const RowSeg rs = row_segment(rows);
    const int64_t row = rs.row, seg = rs.seg;
    const int64_t n = row_bound(row_ends, row, width);
    hoist_args(nseg, seghist, coarse);
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
    // lane t stores bins [16t, 16t+16) as 16-bit counts, and lanes 4c..4c+3 together coarse
    // bin c (fine bins [64c, 64c+64))
    uint32_t c[8];
    uint32_t sum16 = 0;
    const uint4 *h4 = reinterpret_cast<const uint4 *>(hist) + 4 * threadIdx.x;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const uint4 q = h4[v];
        c[2 * v] = q.x | (q.y << 16);
        c[2 * v + 1] = q.z | (q.w << 16);
        sum16 += q.x + q.y + q.z + q.w;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(seghist + (row * nseg + seg) * kBins +
                                           16 * threadIdx.x);
    dst[0] = make_uint4(c[0], c[1], c[2], c[3]);
    dst[1] = make_uint4(c[4], c[5], c[6], c[7]);
    sum16 += lane_xor<1>(sum16);
    sum16 += lane_xor<2>(sum16);
    if ((threadIdx.x & 3) == 0)
        coarse[(row * nseg + seg) * kCoarseBins + (threadIdx.x >> 2)] = (uint16_t)sum16;
}

// One workgroup per row: a row with at most k keys is written whole (all positions, then
// -1); otherwise the threshold bin and every segment's output offsets, in two levels:
//   (a) the 64-bin coarse histograms of all segments give the coarse bin B holding the k-th
//       largest key and the count above B;
//   (b) the 64 fine bins inside B, per segment, give the fine bin b and the count above b;
//   (c) per segment: keys above b = its coarse bins above B + its fine bins in B above b,
//       keys in b = its fine bin b; their exclusive prefix sums are the segment offsets.
// Lane t covers 8 bins (one 16-byte word) t % 8 of segments t / 8 + 128 i. Rows of up to
// 128 segments (every workload here) keep the words of their one block in registers and read
// 256 B per segment once; longer rows read their further blocks again in step (c) (from L2).
constexpr int kSegBlock = kRowThreads / 8;  // segments per block

__device__ __forceinline__ uint32_t sum8(const uint4 &w) {
    return (w.x & 0xFFFFu) + (w.x >> 16) + (w.y & 0xFFFFu) + (w.y >> 16) + (w.z & 0xFFFFu) +
           (w.z >> 16) + (w.w & 0xFFFFu) + (w.w >> 16);
}

// 16-bit count i (0..7) of a word of 8 counts
__device__ __forceinline__ uint32_t count8(const uint4 &w, int i) {
    const uint32_t d = i < 2 ? w.x : i < 4 ? w.y : i < 6 ? w.z : w.w;
    return (i & 1) ? d >> 16 : d & 0xFFFFu;
}

// Word p8 of fine block B (fine bins 64 B .. 64 B + 63) of segment sg, read by the eight
// consecutive lanes of the segment, or zero where the segment has no key in coarse bin B: the
// scorer writes a segment's fine blocks only where its coarse count is nonzero (the rest of a
// reused workspace keeps earlier bytes). `cw` is the lane's word p8 of the segment's coarse
// counts (zero for a segment past the row's keys); the count of bin B is in word B / 8, held
// by the segment's lane p8 = B / 8. Every lane of the wavefront calls it (a lane exchange). The
// load is issued in every lane, at a segment clamped below nseg (in the workspace), so that the
// waits after it count exactly; the words it is not meant to read are masked.
__device__ __forceinline__ uint4 fine_word(const uint4 *fine, int64_t sg, int64_t nseg, uint32_t B,
                                           int p8, const uint4 &cw) {
    const int lane = threadIdx.x & 63;
    const uint32_t cb = (uint32_t)__shfl((int)count8(cw, (int)(B & 7)), (lane & ~7) | (int)(B >> 3));
    const uint4 w = fine[(sg < nseg ? sg : nseg - 1) * (kBins / 8) + B * 8 + p8];
    return cb != 0 ? w : make_uint4(0, 0, 0, 0);
}

// Sum over the lanes of a wavefront that share t % 8 (lanes t % 8 + 8 j), in every one of
// them, in registers: a DPP rotate by 8 within each row of 16, then the cross-row swaps
// (with the value as both operands, each swap pairs rows 0-1 / 2-3, then halves).
__device__ __forceinline__ uint32_t sum_over_segments_in_wave(uint32_t v) {
    v += __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xf, 0xf, false);  // row_ror:8
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = r[0] + r[1];
    const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return h[0] + h[1];
}

// Sum over the 8 consecutive lanes of one segment, in all of them: DPP quad permutes (xor 1,
// xor 2), then the mirror within each half row.
__device__ __forceinline__ uint32_t sum_over_parts(uint32_t v) {
    v += __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
    v += __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
    v += __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xf, 0xf, false);  // row_half_mirror
    return v;
}

// The bin (0..63, counted from the top) holding the k-th largest of 64 descending counts held
// one per lane of wavefront 0, with the count above it; run by wavefront 0 only.
__device__ __forceinline__ void find_in_64(uint32_t c, int k, uint32_t *bin, int *above,
                                           uint32_t *count) {
    const int lane = threadIdx.x & 63;
    const int incl = wave_incl_scan((int)c);
    const int before = incl - (int)c;
    if (before < k && incl >= k) {
        *bin = (uint32_t)lane;
        *above = before;
        *count = c;
    }
}

__global__ __launch_bounds__(kRowThreads) void topk_threshold_kernel(
    const uint16_t *__restrict__ coarse_hist, const uint16_t *__restrict__ fine_hist,
    int64_t nseg, const int32_t *__restrict__ row_ends, int64_t width, int k,
    int32_t *__restrict__ indices, int64_t indices_row_stride, int64_t seg_len,
    RowState *__restrict__ state, uint2 *__restrict__ segoff) {
    __shared__ uint32_t part[kRowThreads / 64][64];
    __shared__ uint32_t seg_above[kMaxRowSegments], seg_in[kMaxRowSegments];
    __shared__ int partials[kRowThreads / 64];
    __shared__ uint32_t found_c, found_f, count_c, count_f;
    __shared__ int above_c, above_f;
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int p8 = t & 7, s0 = t >> 3;
    // the coarse word of this lane's first segment, issued before the row bound is known
    // (every segment < nseg lies in the workspace; those past the row's keys are masked below)
    const uint4 *coarse = reinterpret_cast<const uint4 *>(coarse_hist + row * nseg * kCoarseBins);
    const uint4 *fine = reinterpret_cast<const uint4 *>(fine_hist + row * nseg * kBins);
    const uint4 zero4 = make_uint4(0, 0, 0, 0);
    uint4 cw0 = s0 < nseg ? coarse[s0 * (kCoarseBins / 8) + p8] : zero4;
    const int64_t n = row_bound(row_ends, row, width);
    hoist_args(indices_row_stride, seg_len, state, segoff);
    if (n <= k) {
        int32_t *out = indices + row * indices_row_stride;
        for (int i = t; i < k; i += kRowThreads) out[i] = i < n ? i : -1;
        return;
    }
    const int row_segments = (int)((n + seg_len - 1) / seg_len);
    const int blocks = (row_segments + kSegBlock - 1) / kSegBlock;
    if (s0 >= row_segments) cw0 = zero4;
    if (t == 0) {
        found_c = 0;  // kept only if the counts do not reach k (they always do)
        above_c = 0;
        count_c = 0;
    }

    // (a) coarse totals: bins [8 p8, 8 p8 + 8) summed over this lane's segments, then over the
    // lanes sharing p8 (in the wavefront by shuffles, across wavefronts in LDS)
    uint32_t csum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) csum[e] = count8(cw0, e);
    for (int i = 1; i < blocks; ++i) {
        const int sg = s0 + i * kSegBlock;
        const uint4 w = sg < row_segments ? coarse[sg * (kCoarseBins / 8) + p8] : zero4;
#pragma unroll
        for (int e = 0; e < 8; ++e) csum[e] += count8(w, e);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) csum[e] = sum_over_segments_in_wave(csum[e]);
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[wave][8 * lane + e] = csum[e];
    }
    __syncthreads();
    if (wave == 0) {  // lane l holds coarse bin 63 - l (descending)
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kRowThreads / 64; ++w) c += part[w][63 - lane];
        find_in_64(c, k, &found_c, &above_c, &count_c);
    }
    __syncthreads();
    const uint32_t B = 63u - found_c;  // coarse bin, in ascending order

    // (b) fine bins inside B: word p8 of segment sg covers fine bins 64 B + 8 p8 .. + 8
    const uint4 fw0 = fine_word(fine, s0, nseg, B, p8, cw0);
    uint32_t fsum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) fsum[e] = count8(fw0, e);
    for (int i = 1; i < blocks; ++i) {
        const int sg = s0 + i * kSegBlock;
        const uint4 cw = sg < row_segments ? coarse[sg * (kCoarseBins / 8) + p8] : zero4;
        const uint4 w = fine_word(fine, sg, nseg, B, p8, cw);
#pragma unroll
        for (int e = 0; e < 8; ++e) fsum[e] += count8(w, e);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) fsum[e] = sum_over_segments_in_wave(fsum[e]);
    if (t == 0) {
        found_f = 0;
        above_f = 0;
        count_f = 0;
    }
    __syncthreads();  // part[] is rewritten below
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[wave][8 * lane + e] = fsum[e];
    }
    __syncthreads();
    if (wave == 0) {
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kRowThreads / 64; ++w) c += part[w][63 - lane];
        find_in_64(c, k - above_c, &found_f, &above_f, &count_f);
    }
    __syncthreads();
    const uint32_t f = 63u - found_f;          // fine bin inside B, ascending
    const uint32_t bin = B * 64 + f;           // threshold bin of the 4096

    // (c) per segment: coarse bins above B, fine bins in B above f, and fine bin f
    for (int i = 0; i < blocks; ++i) {
        const int sg = s0 + i * kSegBlock;
        uint4 cw = cw0, fw = fw0;
        if (i > 0) {
            cw = sg < row_segments ? coarse[sg * (kCoarseBins / 8) + p8] : zero4;
            fw = fine_word(fine, sg, nseg, B, p8, cw);
        }
        uint32_t up = 0, in = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b8 = 8u * p8 + e;
            up += b8 > B ? count8(cw, e) : 0u;
            up += b8 > f ? count8(fw, e) : 0u;
            in += b8 == f ? count8(fw, e) : 0u;
        }
        up = sum_over_parts(up);
        in = sum_over_parts(in);
        if (p8 == 0 && sg < row_segments) {
            seg_above[sg] = up;
            seg_in[sg] = in;
        }
    }
    __syncthreads();
    const uint32_t my_above = t < row_segments ? seg_above[t] : 0u;
    const uint32_t my_in = t < row_segments ? seg_in[t] : 0u;
    const int ia = scan_block<kRowThreads>((int)my_above, partials);
    const int ic = scan_block<kRowThreads>((int)my_in, partials);
    if (t < row_segments)
        segoff[row * nseg + t] = make_uint2((uint32_t)ia - my_above, (uint32_t)ic - my_in);
    if (t == 0) {
        const int above = above_c + above_f;
        RowState &st = state[row];
        st.bin = bin;
        st.above = above;
        st.remaining = k - above;
        st.n_cand = count_f;
    }
}

// Keys [lo, hi) of a row held by one workgroup of kTopkThreads lanes, in chunks of 4096 (16 per
// lane, in registers). The caller has loaded the first chunk (`raw`, bounded by `hi` or by the
// row's width: keys past `hi` are masked here). Positions of keys above bin `bin` go to the output
// and (key, position) pairs inside it to the candidate list, after the segment's offsets `off`
// and the earlier chunks' keys (lane counts and a workgroup prefix sum place every key).
constexpr int kCollectPer = 16;
// VEC = 16: rows of whole 16-key runs (width a multiple of 16, 16-byte aligned rows): every lane
// loads one run -- a lane at or past the row's width the row's last run instead, whose keys the
// caller masks (they lie past `bound`) -- so the loads carry no condition and the waits after
// them count exactly. VEC = 4: 16-byte loads for runs below `bound`, single keys for a run it
// cuts. VEC = 1: single keys.
template <int VEC>
__device__ __forceinline__ void load_keys16(float (&raw)[kCollectPer], const float *x,
                                            int64_t first, int64_t bound, int64_t width) {
    if constexpr (VEC == 16) {
        const int64_t at = first < width ? first : width - kCollectPer;
#pragma unroll
        for (int j = 0; j < kCollectPer; j += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(x + at + j);
            raw[j] = v.x;
            raw[j + 1] = v.y;
            raw[j + 2] = v.z;
            raw[j + 3] = v.w;
        }
    } else if (VEC == 4 && first + kCollectPer <= bound) {
#pragma unroll
        for (int j = 0; j < kCollectPer; j += 4) {
            const float4 v = *reinterpret_cast<const float4 *>(x + first + j);
            raw[j] = v.x;
            raw[j + 1] = v.y;
            raw[j + 2] = v.z;
            raw[j + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kCollectPer; ++j) raw[j] = first + j < bound ? x[first + j] : 0.f;
    }
}

// (a & m) | (b & ~m) as one bitfield select. Written as the instruction itself: as plain
// selects, the tree in pick16 is recognised as an indexed read of the register array, which
// the compiler then places in scratch memory.
__device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
}

// raw[j] for a per-lane j < 16: a tree of 15 bitfield selects on the bits of j.
__device__ __forceinline__ float pick16(const float (&raw)[kCollectPer], uint32_t j) {
    static_assert(kCollectPer == 16, "four levels");
    uint32_t a[8], b[4], c[2];
    const uint32_t m0 = 0u - (j & 1u), m1 = 0u - ((j >> 1) & 1u), m2 = 0u - ((j >> 2) & 1u),
                   m3 = 0u - ((j >> 3) & 1u);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        a[i] = bit_select(m0, __float_as_uint(raw[2 * i + 1]), __float_as_uint(raw[2 * i]));
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = bit_select(m1, a[2 * i + 1], a[2 * i]);
#pragma unroll
    for (int i = 0; i < 2; ++i) c[i] = bit_select(m2, b[2 * i + 1], b[2 * i]);
    return __uint_as_float(bit_select(m3, c[1], c[0]));
}

// The float of an order key (the inverse of order_key on keys of non-NaN floats; +0 for the
// key of zero).
__device__ __forceinline__ float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The threshold bin as two float bounds: a logit f is above the bin when f >= hi and inside it
// when lo <= f < hi. Float comparison agrees with the order keys here, signed zeros included:
// order_key gives -0 the key of +0, and IEEE comparison takes -0 equal to +0. A bin holding a
// finite logit lies between the keys of -FLT_MAX and +inf, so both bounds are numbers (the
// upper one +inf for the bin of the largest finite values, above which nothing lies).
struct BinBounds {
    float lo, hi;
    __device__ __forceinline__ explicit BinBounds(uint32_t bin)
        : lo(key_float(bin << kBinShift)), hi(key_float((bin + 1) << kBinShift)) {}
};

// Bit j of `above` / `in`: key j of the lane's 16 (position first + j) lies above the threshold
// bin / inside it; keys at or past `bound` (live = bound - first of them are live) in neither.
struct Masks16 {
    uint32_t above, in;
};
__device__ __forceinline__ Masks16 classify16(const float (&raw)[kCollectPer], int64_t live,
                                              const BinBounds &b) {
    Masks16 m{0u, 0u};
    if (live <= 0) return m;  // a wavefront with no live key skips the work
#pragma unroll
    for (int j = 0; j < kCollectPer; ++j) {
        const float f = raw[j];
        m.above |= f >= b.hi ? 1u << j : 0u;
        m.in |= (f >= b.lo && f < b.hi) ? 1u << j : 0u;
    }
    const uint32_t lm = live >= kCollectPer ? 0xFFFFu : (1u << live) - 1u;
    m.above &= lm;
    m.in &= lm;
    return m;
}


// Positions of the lane's keys above the bin to out[pa], out[pa + 1], .. (while below `cap`),
// in ascending order: one step per set bit.
__device__ __forceinline__ void write_above(uint32_t mask, int64_t first, uint32_t pa,
                                            uint32_t cap, int32_t *out) {
    for (; mask; mask &= mask - 1u, ++pa)
        if (pa < cap) out[pa] = (int32_t)(first + __builtin_ctz(mask));
}

// Keys [lo, hi) of a row held by one workgroup of kTopkThreads lanes, in chunks of 4096 (16 per
// lane, in registers). The caller has loaded the first chunk (`raw`, bounded by `hi` or by the
// row's width: keys past `hi` are masked here). Positions of keys above bin `bin` go to the output
// and (key, position) pairs inside it to the candidate list, after the segment's offsets `off`
// and the earlier chunks' keys (lane counts and a workgroup prefix sum place every key).
template <int VEC, bool NEXT = false>
__device__ __forceinline__ void collect_segment(float (&raw)[kCollectPer], const float *x,
                                                int64_t lo, int64_t hi, int64_t width, uint32_t bin,
                                                uint32_t above, uint2 off, int32_t *out,
                                                uint2 *cand, int *partials,
                                                const float *next = nullptr) {
    constexpr int kChunk = kCollectPer * kTopkThreads;
    const BinBounds bb(bin);
    uint32_t base_above = off.x, base_in = off.y;
    for (int64_t cbase = lo; cbase < hi; cbase += kChunk) {
        const int64_t first = cbase + (int64_t)threadIdx.x * kCollectPer;
        if (cbase != lo) {
            if (NEXT && cbase == lo + kChunk) {  // NEXT: the second chunk, loaded by the caller
#pragma unroll
                for (int j = 0; j < kCollectPer; ++j) raw[j] = next[j];
            } else {
                load_keys16<VEC>(raw, x, first, hi, width);
            }
        }
        const Masks16 m = classify16(raw, hi - first, bb);
        loads_done();
        const int mine = __builtin_popcount(m.above) | (__builtin_popcount(m.in) << 16);
        const int incl = scan_block<kTopkThreads>(mine, partials);
        // the keys' last use comes before any store: a use of a loaded register after a store
        // makes the compiler wait for every store in flight as well (the counter it waits on
        // counts both)
        // one step per key inside the bin (few per lane), not one per key of the lane
        uint32_t pc = base_in + ((incl - mine) >> 16);
        for (uint32_t in = m.in; in; in &= in - 1u, ++pc) {
            const uint32_t j = __builtin_ctz(in);
            if (pc < (uint32_t)kCandCap)
                cand[pc] = make_uint2(order_key(pick16(raw, j)), (uint32_t)(first + j));
        }
        write_above(m.above, first, base_above + ((incl - mine) & 0xFFFF), above, out);
        // the chunk's totals are the sum of the wave totals the scan left in `partials`
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kTopkThreads / 64; ++w) tot += partials[w];
        base_above += (uint32_t)(tot & 0xFFFF);
        base_in += (uint32_t)(tot >> 16);
        if (cbase + kChunk < hi) __syncthreads();  // `partials` is written again by the next scan
    }
}

template <int VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_collect_kernel(
    const float *__restrict__ logits, int64_t logits_row_stride, int64_t width, int64_t seg_len,
    int64_t rows, const int32_t *__restrict__ row_ends, const RowState *__restrict__ state,
    int64_t nseg, const uint2 *__restrict__ segoff, uint2 *__restrict__ cand_all, int k,
    int32_t *__restrict__ indices, int64_t indices_row_stride) {
    __shared__ int partials[kTopkThreads / 64];
    const RowSeg rs = row_segment(rows);
    const int64_t row = rs.row, seg = rs.seg;
    const float *x = logits + row * logits_row_stride;
    const int64_t lo = seg * seg_len;
    // Issued at once, in this order: the row bound and threshold state (scalar loads), the
    // first chunk of keys -- before either arrives: every key below the row's width is in
    // bounds and keys past the row bound are masked -- and the other arguments. The
    // compiler-only fence keeps the loads above the early returns (it emits nothing).
    const int64_t n = row_bound(row_ends, row, width);
    const RowState st = state[row];
    float raw[kCollectPer];
    load_keys16<VEC>(raw, x, lo + (int64_t)threadIdx.x * kCollectPer,
                     lo + seg_len < width ? lo + seg_len : width, width);
    asm volatile("" ::: "memory");
    hoist_args(nseg, segoff, cand_all, k, indices, indices_row_stride);
    if (n <= k) return;
    if (lo >= n) return;
    const int64_t hi = lo + seg_len < n ? lo + seg_len : n;
    collect_segment<VEC>(raw, x, lo, hi, width, st.bin, (uint32_t)st.above, segoff[row * nseg + seg],
                         indices + row * indices_row_stride, cand_all + row * kCandCap,
                         partials);
}

// Steps 2 and 3 in one kernel, for rows of at most kFusedSegments segments (segments x rows
// workgroups, or, with CH = 2, pairs of segments x rows): every workgroup of a row finds the
// row's threshold bin and its own segment's offsets from the row's histograms as
// topk_threshold does (its two levels, the same sums), reading 2 x 128 B per segment of the
// row, then collects its segment (pair). The row's first segment also stores the threshold
// state for step 4, or, for a row of at most k keys, the whole output. Pairs halve the
// workgroups that large batches of uneven rows dispatch, most of them past the rows' keys (a
// row past its keys costs one round trip per workgroup), and the threshold work per key.
constexpr int kFusedSegments = 64;
static_assert(kFusedSegments == 64 && kTopkThreads == 256, "lane t covers word t % 8 of two segments");

template <int VEC, int CH>
__global__ __launch_bounds__(kTopkThreads) void topk_threshold_collect_kernel(
    const float *__restrict__ logits, int64_t logits_row_stride, int64_t width,
    const int32_t *__restrict__ row_ends, const uint16_t *__restrict__ coarse_hist, int rows,
    int nseg, int seg_len, int k, const uint16_t *__restrict__ fine_hist,
    int32_t *__restrict__ indices, int64_t indices_row_stride, RowState *__restrict__ state,
    uint2 *__restrict__ cand_all) {
    __shared__ int partials[kTopkThreads / 64];
    __shared__ uint32_t part[kTopkThreads / 64][64], part_f[kTopkThreads / 64][64];
    __shared__ uint32_t seg_above[kFusedSegments], seg_in[kFusedSegments];
    static_assert(CH == 1 || CH == 2, "one or two segments per workgroup");
    const RowSeg rs = row_segment(rows);
    const int64_t row = rs.row, seg = rs.seg * CH;  // the workgroup's first segment
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int p8 = t & 7, s0 = t >> 3;  // word p8 of segments s0 and s0 + 32
    const float *x = logits + row * logits_row_stride;
    const int64_t lo = seg * (int64_t)seg_len;
    const uint4 zero4 = make_uint4(0, 0, 0, 0);

    // Issued at once: the row bound, the coarse words of the row's segments (every segment
    // below nseg lies in the workspace; those past the row's keys are masked below) and the
    // other arguments. The segment's keys go out once the bound shows the segment holds keys
    // of the row, and arrive while the fine histogram words are fetched: loading them before
    // that, for every segment of every row, read tens of MB of logits past the rows' ends on
    // ragged workloads.
    // (Loads are issued in every lane, at segments clamped below nseg, and masked at their
    // use: conditional loads, or registers of loads in flight written over, make the compiler
    // wait for every load in flight, the segment's keys included.)
    const uint4 *coarse = reinterpret_cast<const uint4 *>(coarse_hist + row * nseg * kCoarseBins);
    const int sa = s0 < nseg ? s0 : nseg - 1, sb = s0 + 32 < nseg ? s0 + 32 : nseg - 1;
    const uint4 cl0 = coarse[sa * (kCoarseBins / 8) + p8];
    const uint4 cl1 = coarse[sb * (kCoarseBins / 8) + p8];
    const int32_t end = row_ends[row];
    hoist_args(fine_hist, indices, indices_row_stride, state, cand_all);
    // nothing that needs the row bound moves above the loads: the coarse words leave in the
    // bound's round trip instead of one round trip after it
    __builtin_amdgcn_sched_barrier(0);
    const int64_t n = end < 0 ? 0 : (end > width ? width : (int64_t)end);
    if (n <= k) {
        if (seg == 0) {
            int32_t *out = indices + row * indices_row_stride;
            for (int i = t; i < k; i += kTopkThreads) out[i] = i < n ? i : -1;
        }
        keep_loaded(cl0.x);
        keep_loaded(cl1.x);
        return;
    }
    if (lo >= n) return;
    const int64_t hi = lo + (int64_t)CH * seg_len < n ? lo + (int64_t)CH * seg_len : n;
    float raw[kCollectPer], raw2[CH == 2 ? kCollectPer : 1];
    load_keys16<VEC>(raw, x, lo + (int64_t)t * kCollectPer, hi, width);
    if constexpr (CH == 2)  // the second chunk of keys too, in the same round trip
        load_keys16<VEC>(raw2, x, lo + (int64_t)(kTopkThreads + t) * kCollectPer, hi, width);
    const int row_segments = (int)((n + seg_len - 1) / seg_len);
    const uint4 cw0 = s0 < row_segments ? cl0 : zero4;
    const uint4 cw1 = s0 + 32 < row_segments ? cl1 : zero4;

    // (a) coarse totals: bins [8 p8, 8 p8 + 8) over this lane's segments, then over the lanes
    // sharing p8 (in the wavefront by lane swaps, across wavefronts in LDS); after one barrier
    // every wavefront reads the four partial rows and finds the bin itself (lane l: coarse bin
    // 63 - l, descending), so no wavefront waits on another's result
    uint32_t csum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) csum[e] = sum_over_segments_in_wave(count8(cw0, e) + count8(cw1, e));
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[wave][8 * lane + e] = csum[e];
    }
    __syncthreads();
    uint32_t cc = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) cc += part[w][63 - lane];
    const Found64 fc = find_in_64_wave(cc, k);
    const uint32_t B = 63u - (uint32_t)fc.lane;  // coarse bin, in ascending order

    // (b) fine bins inside B: word p8 of segment sg covers fine bins 64 B + 8 p8 .. + 8
    const uint4 *fine = reinterpret_cast<const uint4 *>(fine_hist + row * nseg * kBins);
    const uint4 fw0 = fine_word(fine, s0, nseg, B, p8, cw0);
    const uint4 fw1 = fine_word(fine, s0 + 32, nseg, B, p8, cw1);
    uint32_t fsum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) fsum[e] = sum_over_segments_in_wave(count8(fw0, e) + count8(fw1, e));
    if (lane < 8) {  // (a row of its own: the coarse rows may still be read)
#pragma unroll
        for (int e = 0; e < 8; ++e) part_f[wave][8 * lane + e] = fsum[e];
    }
    __syncthreads();
    uint32_t fc2 = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) fc2 += part_f[w][63 - lane];
    const Found64 ff = find_in_64_wave(fc2, k - fc.before);
    const uint32_t f = 63u - (uint32_t)ff.lane;  // fine bin inside B, ascending
    const uint32_t bin = B * 64 + f;             // threshold bin of the 4096
    const int above = fc.before + ff.before;

    // (c) per segment: coarse bins above B, fine bins in B above f, and fine bin f; after one
    // barrier every wavefront takes the exclusive prefix sums over the segments for this
    // workgroup's segment itself
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint4 &cw = h ? cw1 : cw0;
        const uint4 &fw = h ? fw1 : fw0;
        uint32_t up = 0, in = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t b8 = 8u * p8 + e;
            up += b8 > B ? count8(cw, e) : 0u;
            up += b8 > f ? count8(fw, e) : 0u;
            in += b8 == f ? count8(fw, e) : 0u;
        }
        up = sum_over_parts(up);
        in = sum_over_parts(in);
        if (p8 == 0) {
            seg_above[s0 + 32 * h] = up;  // zero for segments past the row's keys
            seg_in[s0 + 32 * h] = in;
        }
    }
    __syncthreads();
    const int sa_ = (int)seg_above[lane], sc_ = (int)seg_in[lane];
    const int ia = wave_incl_scan(sa_), ic = wave_incl_scan(sc_);
    const uint2 my_off = make_uint2((uint32_t)__builtin_amdgcn_readlane(ia - sa_, (int)seg),
                                    (uint32_t)__builtin_amdgcn_readlane(ic - sc_, (int)seg));
    if (seg == 0 && t == 0) {
        RowState &st = state[row];
        st.bin = bin;
        st.above = above;
        st.remaining = k - above;
        st.n_cand = ff.count;
    }
    collect_segment<VEC, CH == 2>(raw, x, lo, hi, width, bin, (uint32_t)above, my_off,
                                  indices + row * indices_row_stride, cand_all + row * kCandCap,
                                  partials, raw2);
}


// Composites held in registers, S per lane: lane t's i-th is candidate t + i * kSelectThreads
// of m.
template <int S>
struct RegCandidates {
    uint64_t c[S];
    int m;
    template <typename F>
    __device__ __forceinline__ void for_each(F &&f) const {
#pragma unroll
        for (int i = 0; i < S; ++i)
            if ((int)threadIdx.x + i * kSelectThreads < m) f(c[i]);
    }
};

__global__ __launch_bounds__(kSelectThreads) void topk_select_kernel(
    const uint2 *__restrict__ cand_all, const RowState *__restrict__ state,
    const int32_t *__restrict__ row_ends, int64_t width, int k, int32_t *__restrict__ indices,
    int64_t indices_row_stride, const float *__restrict__ logits, int64_t logits_row_stride) {
    __shared__ uint64_t cands[kCandCap];
    __shared__ SelectShared<> sh;
    const int64_t row = blockIdx.x;
    // the first kSpec candidates, loaded before their count is known (the list always has
    // kCandCap slots; slots past the count are ignored)
    // Issued at once (the scheduling barrier keeps the bound's arithmetic after every load):
    // the speculative candidates, the row bound and state (scalar loads) and the other
    // arguments.
    constexpr int kSpec = 4;
    const uint2 *cand = cand_all + row * kCandCap;
    uint2 pre[kSpec];
#pragma unroll
    for (int i = 0; i < kSpec; ++i) pre[i] = cand[threadIdx.x + i * kSelectThreads];
    const RowState st = state[row];
    const int32_t end = row_ends[row];
    hoist_args(logits, logits_row_stride);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t n = end < 0 ? 0 : (end > width ? width : end);
    if (n <= k) {
#pragma unroll
        for (int i = 0; i < kSpec; ++i) {
            keep_loaded(pre[i].x);
            keep_loaded(pre[i].y);
        }
        keep_loaded(st.bin);
        keep_loaded((uint32_t)st.above);
        keep_loaded((uint32_t)st.remaining);
        keep_loaded(st.n_cand);
        return;
    }
    const float *x = logits + row * logits_row_stride;
    const uint32_t bin = st.bin, ncand = st.n_cand;
    const int remaining = st.remaining;
    if (remaining <= 0 || remaining > k) return;
    int32_t *out = indices + row * indices_row_stride + st.above;
    int pos_bits = 1;
    while (pos_bits < 31 && ((int64_t)1 << pos_bits) < n) ++pos_bits;
    const int bits = 20 + pos_bits;
    if (ncand <= (uint32_t)(kSpec * kSelectThreads)) {  // all of them already in registers
        RegCandidates<kSpec> rc;
#pragma unroll
        for (int i = 0; i < kSpec; ++i) rc.c[i] = composite(pre[i].x, pre[i].y, pos_bits);
        rc.m = (int)ncand;
        select_smallest(rc, remaining, bits, pos_bits, out, sh);
    } else if (ncand <= (uint32_t)kCandCap) {
#pragma unroll
        for (int i = 0; i < kSpec; ++i) {
            const int j = threadIdx.x + i * kSelectThreads;
            if (j < (int)ncand) cands[j] = composite(pre[i].x, pre[i].y, pos_bits);
        }
        for (int j = threadIdx.x + kSpec * kSelectThreads; j < (int)ncand; j += kSelectThreads) {
            const uint2 e = cand[j];
            cands[j] = composite(e.x, e.y, pos_bits);
        }
        __syncthreads();
        select_smallest(LdsCandidates<>{cands, (int)ncand}, remaining, bits, pos_bits, out, sh);
    } else {
        select_smallest(RowBin<>{x, n, bin, pos_bits}, remaining, bits, pos_bits, out, sh);
    }
}

// Steps 2 to 4 in one workgroup per row, for rows of at most kRowTopkWidth keys and 64
// segments, with the whole row in the workgroup's registers (16 keys per lane). The threshold
// bin in the two levels of topk_threshold: every wavefront sums the coarse counts of all the
// row's segments itself (so none waits for another), and the fine counts inside the coarse bin
// come from the row's own keys (LDS counts). Then the keys are classified once: positions above
// the bin go to the output, in ascending order, and (key, position) pairs inside it to LDS,
// placed by a workgroup prefix sum. The candidates are taken whole when they all fit, selected
// by one wavefront when there are at most 64 of them (the usual case), and by the radix select
// of step 4 otherwise. Four workgroup barriers in all. Measured, one workgroup per row wins
// only while a row is one chunk of 8192 keys: classifying 32K-key rows on one compute unit
// took longer than the two segmented launches (decode workload step 49 -> 57 us).
constexpr int kRowTopkWidth = 8192;
static_assert(kSelectThreads == 512 && kFusedSegments == 64, "lane l covers word l % 8 of segments l / 8 + 8 i");
static_assert(kRowTopkWidth == kCollectPer * kSelectThreads, "a row is one chunk, all in registers");
static_assert(kRowTopkWidth <= kCandCap, "every key of a row fits the LDS candidate list");

template <int VEC>
__global__ __launch_bounds__(kSelectThreads) void topk_row_kernel(
    const int32_t *__restrict__ row_ends, const uint16_t *__restrict__ coarse_hist,
    const float *__restrict__ logits, int64_t logits_row_stride, int64_t width, int nseg,
    int seg_len, int k, int32_t *__restrict__ indices, int64_t indices_row_stride) {
    constexpr int kWaves = kSelectThreads / 64;
    __shared__ uint64_t cands[kCandCap];
    __shared__ SelectShared<> sh;
    __shared__ uint32_t part[kWaves][64];
    __shared__ uint32_t fine_count[64];
    __shared__ int wave_total[kWaves];
    const int64_t row = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int p8 = lane & 7, s8 = lane >> 3;  // word p8 of segments s8 + 8 i
    const int64_t first = (int64_t)t * kCollectPer;

    // Issued at once: the coarse words of all the row's segments in every wavefront (segments
    // clamped below nseg, in the workspace; those past the row's keys are masked at their use),
    // with whole 16-key runs the row's keys up to its width, the row bound and the other
    // arguments. Unconditional loads masked at use keep the compiler's waits exact; the
    // scheduling barrier keeps everything that needs the bound below the loads, so they all
    // leave in one round trip, and the first workgroup barrier (the fine counts' zeroing)
    // passes while they are in flight.
    const uint4 *coarse = reinterpret_cast<const uint4 *>(coarse_hist + row * nseg * kCoarseBins);
    uint4 cl[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int sg = s8 + 8 * i;
        cl[i] = coarse[(sg < nseg ? sg : nseg - 1) * (kCoarseBins / 8) + p8];
    }
    const float *x = logits + row * logits_row_stride;
    float raw[kCollectPer];
    if constexpr (VEC == 16) load_keys16<VEC>(raw, x, first, width, width);
    const int32_t end = row_ends[row];
    hoist_args(indices, indices_row_stride);
    if (t < 64) fine_count[t] = 0;
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // 1: fine_count is zero
    const int64_t n = end < 0 ? 0 : (end > width ? width : (int64_t)end);
    int32_t *out = indices + row * indices_row_stride;
    if (n <= k) {
        for (int i = t; i < k; i += kSelectThreads) out[i] = i < n ? i : -1;
#pragma unroll
        for (int i = 0; i < 8; ++i) keep_loaded(cl[i].x);
        if constexpr (VEC == 16) keep_loaded(__float_as_uint(raw[0]));
        return;
    }
    if constexpr (VEC != 16) load_keys16<VEC>(raw, x, first, n, width);
    const int row_segments = (int)((n + seg_len - 1) / seg_len);
    // wavefronts past the row's keys skip the per-key steps (still at every barrier, as the
    // radix select needs them), so that a short row costs its own wavefronts' issue time only
    const bool has_keys = (int64_t)wave * (64 * kCollectPer) < n;

    // (a) coarse totals, per wavefront: bins 8 p8 + e summed over the lane's segments and then
    // over the lanes sharing p8, turned to one bin per lane (descending) through the
    // wavefront's own LDS row, and the coarse bin B holding the k-th largest key
    uint32_t csum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t v = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) v += s8 + 8 * i < row_segments ? count8(cl[i], e) : 0u;
        csum[e] = sum_over_segments_in_wave(v);
    }
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) part[wave][8 * lane + e] = csum[e];
    }
    __builtin_amdgcn_wave_barrier();
    const Found64 fc = find_in_64_wave(part[wave][63 - lane], k);
    const uint32_t B = 63u - (uint32_t)fc.lane;  // ascending coarse bin

    // (b) fine counts inside B from the keys in registers, then the fine bin f in every
    // wavefront
    if (has_keys) {
        const int64_t live = n - first;
#pragma unroll
        for (int j = 0; j < kCollectPer; ++j) {
            const uint32_t u = order_key(raw[j]);
            if (j < live && (u >> (kBinShift + 6)) == B)
                atomicAdd(&fine_count[(u >> kBinShift) & 63u], 1u);
        }
    }
    __syncthreads();  // 2: the fine counts are complete
    const Found64 ff = find_in_64_wave(fine_count[63 - lane], k - fc.before);
    const uint32_t bin = B * 64 + (63u - (uint32_t)ff.lane);
    const int above = fc.before + ff.before;
    const int m = (int)ff.count;  // keys inside the bin
    const int r = k - above;      // of which the r largest are taken (1 <= r <= m)
    int pos_bits = 1;
    while (pos_bits < 31 && ((int64_t)1 << pos_bits) < n) ++pos_bits;

    // (c) the keys once: lane counts and a workgroup prefix sum place every key (the
    // wavefronts past the keys have none and come after every wavefront that has some)
    Masks16 mk{0u, 0u};
    int mine = 0, incl = 0;
    if (has_keys) {
        mk = classify16(raw, n - first, BinBounds(bin));
        mine = __builtin_popcount(mk.above) | (__builtin_popcount(mk.in) << 16);
        incl = wave_incl_scan(mine);
        if (lane == 63) wave_total[wave] = incl;
    }
    __syncthreads();  // 3: the wavefront totals
    if (has_keys) {
        int excl = incl - mine;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) excl += w < wave ? wave_total[w] : 0;
        uint32_t pc = (uint32_t)excl >> 16;
        if (r == m) {  // every key inside the bin is taken
            for (uint32_t in = mk.in; in; in &= in - 1u, ++pc)
                if (above + (int)pc < k) out[above + pc] = (int32_t)(first + __builtin_ctz(in));
        } else {
            for (uint32_t in = mk.in; in; in &= in - 1u, ++pc) {
                const uint32_t j = __builtin_ctz(in);
                cands[pc] = composite(order_key(pick16(raw, j)), (uint32_t)(first + j), pos_bits);
            }
        }
        write_above(mk.above, first, (uint32_t)excl & 0xFFFFu, (uint32_t)above, out);
    }
    if (r == m) return;
    __syncthreads();  // 4: the candidates are in LDS

    // (d) the r smallest composites inside the bin
    const int bits = 20 + pos_bits;
    if (m <= 64) {
        if (wave == 0) {
            const uint64_t c = lane < m ? cands[lane] : ~(uint64_t)0;
            const uint64_t taken = wave_select_smallest(c, m, r, bits);
            if ((taken >> lane) & 1ull) {
                const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(taken >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)taken, 0u));
                out[above + slot] = (int32_t)(c & (((uint64_t)1 << pos_bits) - 1));
            }
        }
    } else {
        select_smallest(LdsCandidates<>{cands, m}, r, bits, pos_bits, out + above, sh);
    }
}

size_t topk_workspace_bytes(int64_t rows, int64_t width, int) {
    return topk_layout_bytes(rows, topk_nseg(width, topk_segment(rows, width)));
}

// topk_threshold_collect_kernel with CH segments per workgroup, with the widest key loads the
// rows allow.
template <int CH>
static void launch_threshold_collect(bool runs, bool vec, hipStream_t stream, const float *logits,
                                     int64_t logits_row_stride, int64_t width,
                                     const int32_t *row_ends, const TopkWorkspace &ws, int64_t rows,
                                     int64_t nseg, int64_t seg_len, int k, int32_t *indices,
                                     int64_t indices_row_stride) {
    const dim3 grid((unsigned)(rows * ((nseg + CH - 1) / CH))), block(kTopkThreads);
    if (runs)
        hipLaunchKernelGGL((topk_threshold_collect_kernel<16, CH>), grid, block, 0, stream, logits,
                           logits_row_stride, width, row_ends, ws.coarse, (int)rows, (int)nseg,
                           (int)seg_len, k, ws.seghist, indices, indices_row_stride, ws.state,
                           ws.cand);
    else if (vec)
        hipLaunchKernelGGL((topk_threshold_collect_kernel<4, CH>), grid, block, 0, stream, logits,
                           logits_row_stride, width, row_ends, ws.coarse, (int)rows, (int)nseg,
                           (int)seg_len, k, ws.seghist, indices, indices_row_stride, ws.state,
                           ws.cand);
    else
        hipLaunchKernelGGL((topk_threshold_collect_kernel<1, CH>), grid, block, 0, stream, logits,
                           logits_row_stride, width, row_ends, ws.coarse, (int)rows, (int)nseg,
                           (int)seg_len, k, ws.seghist, indices, indices_row_stride, ws.state,
                           ws.cand);
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
    // rows of whole 16-key runs (every scorer-made row: its width is a multiple of 64 keys)
    const bool runs = vec && width >= kCollectPer && width % kCollectPer == 0;
    if (nseg <= kFusedSegments && width <= kRowTopkWidth) {
        if (runs)
            hipLaunchKernelGGL(topk_row_kernel<16>, dim3((unsigned)rows), dim3(kSelectThreads), 0,
                               stream, row_ends, ws.coarse, logits, logits_row_stride, width,
                               (int)nseg, (int)seg_len, k, indices, indices_row_stride);
        else if (vec)
            hipLaunchKernelGGL(topk_row_kernel<4>, dim3((unsigned)rows), dim3(kSelectThreads), 0,
                               stream, row_ends, ws.coarse, logits, logits_row_stride, width,
                               (int)nseg, (int)seg_len, k, indices, indices_row_stride);
        else
            hipLaunchKernelGGL(topk_row_kernel<1>, dim3((unsigned)rows), dim3(kSelectThreads), 0,
                               stream, row_ends, ws.coarse, logits, logits_row_stride, width,
                               (int)nseg, (int)seg_len, k, indices, indices_row_stride);
        return hipGetLastError();
    }
    if (nseg <= kFusedSegments) {
        // launches of many more (row, segment) items than about four workgroups per compute
        // unit, of segments of at most one chunk: two segments per workgroup, their keys
        // loaded together (two segments of several chunks each measured slower)
        if (rows * nseg > (int64_t)device_cus() * 4 && seg_len <= kCollectPer * kTopkThreads)
            launch_threshold_collect<2>(runs, vec, stream, logits, logits_row_stride, width,
                                        row_ends, ws, rows, nseg, seg_len, k, indices,
                                        indices_row_stride);
        else
            launch_threshold_collect<1>(runs, vec, stream, logits, logits_row_stride, width,
                                        row_ends, ws, rows, nseg, seg_len, k, indices,
                                        indices_row_stride);
        hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)rows), dim3(kSelectThreads), 0,
                           stream, ws.cand, ws.state, row_ends, width, k, indices,
                           indices_row_stride, logits, logits_row_stride);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(topk_threshold_kernel, dim3((unsigned)rows), dim3(kRowThreads), 0, stream,
                       ws.coarse, ws.seghist, nseg, row_ends, width, k, indices,
                       indices_row_stride, seg_len, ws.state, ws.segoff);
    if (runs)
        hipLaunchKernelGGL(topk_collect_kernel<16>, grid, block, 0, stream, logits,
                           logits_row_stride, width, seg_len, rows, row_ends, ws.state, nseg,
                           ws.segoff, ws.cand, k, indices, indices_row_stride);
    else if (vec)
        hipLaunchKernelGGL(topk_collect_kernel<4>, grid, block, 0, stream, logits,
                           logits_row_stride, width, seg_len, rows, row_ends, ws.state, nseg,
                           ws.segoff, ws.cand, k, indices, indices_row_stride);
    else
        hipLaunchKernelGGL(topk_collect_kernel<1>, grid, block, 0, stream, logits,
                           logits_row_stride, width, seg_len, rows, row_ends, ws.state, nseg,
                           ws.segoff, ws.cand, k, indices, indices_row_stride);
    hipLaunchKernelGGL(topk_select_kernel, dim3((unsigned)rows), dim3(kSelectThreads), 0, stream,
                       ws.cand, ws.state, row_ends, width, k, indices, indices_row_stride, logits,
                       logits_row_stride);
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
        hipLaunchKernelGGL(topk_hist_kernel<4>, grid, block, 0, stream, logits,
                           logits_row_stride, width, seg_len, rows, row_ends, k, nseg,
                           ws.seghist, ws.coarse);
    else
        hipLaunchKernelGGL(topk_hist_kernel<1>, grid, block, 0, stream, logits,
                           logits_row_stride, width, seg_len, rows, row_ends, k, nseg,
                           ws.seghist, ws.coarse);
    return launch_topk_after_histograms(logits, rows, width, logits_row_stride, row_ends, k,
                                        indices, indices_row_stride, workspace, nseg, seg_len,
                                        stream);
}

// The workspace of the allocation-free top-k (dsaidx_topk_noalloc): a file-scope device
// array, one copy per device, held until the process ends. In host code its name stands for
// no device address; the address comes from hipGetSymbolAddress, taken once per device with
// that device current and kept in scratch_address_of.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

static std::mutex scratch_mutex;
static void *scratch_address_of[kMaxScratchDevices];

hipError_t static_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_address_of[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_address_of[dev] = p;
    }
    *out = scratch_address_of[dev];
    return hipSuccess;
}

}  // namespace dsaidx
