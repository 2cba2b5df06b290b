// Workgroup scans and the radix select in LDS shared by the top-k and the DCP merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

constexpr int kSelectThreads = 512;
constexpr int kRadixBits = 11;
constexpr int kRadixBins = 1 << kRadixBits;

// Inclusive prefix sum over the wavefront on the data-parallel primitives (DPP): shifts by
// 1, 2, 4 and 8 lanes within each row of 16, then row 0's and row 1's totals broadcast
// into the rows above them. All in registers, no LDS round trips.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return x;
}

// Inclusive prefix sum over an NT-lane workgroup; `partials` holds NT / 64 ints. On return
// partials[w] is wavefront w's total (valid until the next call).
template <int NT>
__device__ __forceinline__ int scan_block(int v, int *partials) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_incl_scan(v);
    if (lane == 63) partials[wave] = v;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) before += w < wave ? partials[w] : 0;
    __syncthreads();
    return v + before;
}

struct LdsCandidates {  // composites already in LDS (distinct)
    const uint64_t *c;
    int m;
    template <typename F>
    __device__ __forceinline__ void for_each(F &&f) const {
        for (int j = threadIdx.x; j < m; j += kSelectThreads) f(c[j]);
    }
};

struct SelectShared {
    uint32_t hist[kRadixBins];
    int partials[kSelectThreads / 64];
    uint64_t prefix;
    int below;
    int count;
    uint32_t n_out;
};

// The r-th smallest of the distinct composites (of `bits` significant bits, 1 <= r <= their
// count) that `src` yields, by a most-significant-digit radix select in LDS: exactly r
// composites are <= the returned value. Every lane of the workgroup must call it.
template <typename Source>
__device__ uint64_t select_threshold(const Source &src, int r, int bits, SelectShared &sh) {
    uint64_t prefix = 0;
    int done = 0;  // high composite bits fixed in `prefix`
    uint64_t threshold = ~(uint64_t)0;
    while (done < bits) {
        const int digit = bits - done >= kRadixBits ? kRadixBits : bits - done;
        const int shift = bits - done - digit;
        for (int b = threadIdx.x; b < kRadixBins; b += kSelectThreads) sh.hist[b] = 0;
        __syncthreads();
        const uint64_t want = prefix >> (shift + digit);
        src.for_each([&](uint64_t c) {
            if ((c >> (shift + digit)) == want)
                atomicAdd(&sh.hist[(uint32_t)(c >> shift) & (uint32_t)((1 << digit) - 1)], 1u);
        });
        __syncthreads();
        constexpr int per = kRadixBins / kSelectThreads;  // ascending: lane t owns per*t ..
        int own = 0;
        uint32_t mine[per];
#pragma unroll
        for (int j = 0; j < per; ++j) {
            mine[j] = sh.hist[threadIdx.x * per + j];
            own += (int)mine[j];
        }
        const int incl = scan_block<kSelectThreads>(own, sh.partials);
        int before = incl - own;
#pragma unroll
        for (int j = 0; j < per; ++j) {
            const int c = (int)mine[j];
            if (before < r && before + c >= r) {
                sh.prefix = prefix | ((uint64_t)(threadIdx.x * per + j) << shift);
                sh.below = before;
                sh.count = c;
            }
            before += c;
        }
        __syncthreads();
        prefix = sh.prefix;
        done += digit;
        if (sh.below + sh.count == r) {  // the whole digit bin is taken: stop early
            threshold = prefix | (((uint64_t)1 << shift) - 1);
            break;
        }
        r -= sh.below;
        threshold = prefix;
        __syncthreads();
    }
    return threshold;
}

// Slots for the lanes of a wavefront whose `take` is set (among the active lanes), from the
// counter `n`: one atomic per wavefront, then each lane's rank among the taken lanes.
__device__ __forceinline__ uint32_t wave_slot(bool take, uint32_t *n) {
    const uint64_t mask = __ballot(take);
    uint32_t base = 0;
    if (mask) {
        const int leader = __builtin_ctzll(mask);
        if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(n, (uint32_t)__builtin_popcountll(mask));
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
    }
    return base + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Writes the low `pos_bits` bits (the position) of the r smallest composites to out[0..r),
// in no particular order.
template <typename Source>
__device__ void select_smallest(const Source &src, int r, int bits, int pos_bits, int32_t *out,
                                SelectShared &sh) {
    const uint64_t threshold = select_threshold(src, r, bits, sh);
    if (threadIdx.x == 0) sh.n_out = 0;
    __syncthreads();
    const uint64_t pos_mask = ((uint64_t)1 << pos_bits) - 1;
    src.for_each([&](uint64_t c) {
        const bool take = c <= threshold;
        const uint32_t slot = wave_slot(take, &sh.n_out);
        if (take && slot < (uint32_t)r) out[slot] = (int32_t)(c & pos_mask);
    });
}

}  // namespace dsaidx
