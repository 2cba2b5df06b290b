// Workgroup scans and the radix select in LDS shared by the top-k and the DCP merge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "topk_layout.h"

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

// NT: the workgroup's lanes (every lane takes part)
template <int NT = kSelectThreads>
struct LdsCandidates {  // composites already in LDS (distinct)
    const uint64_t *c;
    int m;
    template <typename F>
    __device__ __forceinline__ void for_each(F &&f) const {
        for (int j = threadIdx.x; j < m; j += NT) f(c[j]);
    }
};

template <int NT = kSelectThreads>
struct SelectShared {
    uint32_t hist[kRadixBins];
    int partials[NT / 64];
    uint64_t prefix;
    int below;
    int count;
    uint32_t n_out, n_tie;
    uint64_t ties[64];  // the composites of the threshold digit (select_smallest)
};

// One digit of the radix select in LDS: among the composites whose bits above `shift + digit`
// equal those of `prefix`, the value d of the next `digit` bits that holds the r-th smallest
// of them (1 <= r <= their count). On return sh.prefix = prefix with d placed at `shift`,
// sh.below = how many of them have a smaller digit, sh.count = how many have d. Every lane of
// the workgroup must call it.
template <typename Source, int NT>
__device__ void radix_digit(const Source &src, uint64_t prefix, int digit, int shift, int r,
                            SelectShared<NT> &sh) {
    for (int b = threadIdx.x; b < kRadixBins; b += NT) sh.hist[b] = 0;
    __syncthreads();
    const uint64_t want = prefix >> (shift + digit);
    src.for_each([&](uint64_t c) {
        if ((c >> (shift + digit)) == want)
            atomicAdd(&sh.hist[(uint32_t)(c >> shift) & (uint32_t)((1 << digit) - 1)], 1u);
    });
    __syncthreads();
    constexpr int per = kRadixBins / NT;  // ascending: lane t owns per*t ..
    int own = 0;
    uint32_t mine[per];
#pragma unroll
    for (int j = 0; j < per; ++j) {
        mine[j] = sh.hist[threadIdx.x * per + j];
        own += (int)mine[j];
    }
    const int incl = scan_block<NT>(own, sh.partials);
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
}

// The r-th smallest of the distinct composites (of `bits` significant bits, 1 <= r <= their
// count) that `src` yields, by a most-significant-digit radix select in LDS: exactly r
// composites are <= the returned value. A caller that has already fixed the top `done` bits
// passes them in `prefix` with r counted among the composites that share them. Every lane of
// the workgroup must call it.
template <typename Source, int NT>
__device__ uint64_t select_threshold(const Source &src, int r, int bits, SelectShared<NT> &sh,
                                     uint64_t prefix = 0, int done = 0) {
    uint64_t threshold = prefix;
    while (done < bits) {
        const int digit = bits - done >= kRadixBits ? kRadixBits : bits - done;
        const int shift = bits - done - digit;
        radix_digit(src, prefix, digit, shift, r, sh);
        prefix = sh.prefix;
        done += digit;
        if (sh.below + sh.count == r) {  // the whole digit bin is taken: stop early
            threshold = prefix | (((uint64_t)1 << shift) - 1);
            break;
        }
        r -= sh.below;
        threshold = prefix;
    }
    return threshold;
}

// Composite of a key inside the threshold bin: smaller for a larger value, and for equal
// values smaller for the lower position; unique per position.
__device__ __forceinline__ uint64_t composite(uint32_t u, uint32_t pos, int pos_bits) {
    return ((uint64_t)(~u & 0xFFFFFu) << pos_bits) | pos;
}

// The lane of a wavefront holding the k-th largest of 64 descending counts (one per lane), the
// count before it and its own count, as wavefront-uniform values. The counts reach k.
struct Found64 {
    int lane, before;
    uint32_t count;
};
__device__ __forceinline__ Found64 find_in_64_wave(uint32_t c, int k) {
    const int incl = wave_incl_scan((int)c);
    const int before = incl - (int)c;
    const uint64_t hit = __ballot(before < k && incl >= k);
    const int L = hit ? __builtin_ctzll(hit) : 63;
    return {L, __builtin_amdgcn_readlane(before, L), (uint32_t)__builtin_amdgcn_readlane((int)c, L)};
}

// Set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
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

// The r smallest of m <= 64 distinct composites (`bits` significant bits), one per lane of a
// wavefront in lanes [0, m): bit by bit from the top, the undecided composites whose bit is 0
// are all taken if they fit in what is left of r, else the search continues among them.
// Returns the mask of the taken lanes.
__device__ __forceinline__ uint64_t wave_select_smallest(uint64_t c, int m, int r, int bits) {
    const int lane = threadIdx.x & 63;
    uint64_t active = __ballot(lane < m), taken = 0;
    for (int b = bits - 1; b >= 0 && r > 0; --b) {
        const uint64_t zeros = active & __ballot(((c >> b) & 1ull) == 0);
        const int nz = __builtin_popcountll(zeros);
        if (nz <= r) {
            taken |= zeros;
            r -= nz;
            active &= ~zeros;
        } else {
            active = zeros;
        }
        if (__builtin_popcountll(active) == r) {
            taken |= active;
            r = 0;
        }
    }
    return taken;
}

// The r smallest of m <= 64 distinct composites c[0..m) (in LDS) to out[0..r), by one
// wavefront's bit-by-bit select; the composite's low `pos_bits` bits are the position written.
__device__ __forceinline__ void wave_select_out(const uint64_t *c, int m, int r, int bits,
                                                int pos_bits, int32_t *out) {
    const int lane = threadIdx.x & 63;
    const uint64_t v = lane < m ? c[lane] : ~(uint64_t)0;
    const uint64_t taken = wave_select_smallest(v, m, r, bits);
    if ((taken >> lane) & 1ull) {
        const uint32_t slot = __builtin_amdgcn_mbcnt_hi(
            (uint32_t)(taken >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)taken, 0u));
        out[slot] = (int32_t)(v & (((uint64_t)1 << pos_bits) - 1));
    }
}

// Writes the low `pos_bits` bits (the position) of the r smallest composites to out[0..r),
// in no particular order. A first digit of the top 8 bits (256 counts, scanned by one
// wavefront) finds the digit d holding the r-th smallest; one pass then takes every composite
// of a smaller digit and gathers those of digit d, and, unless d is taken whole, one wavefront
// selects among them bit by bit: four workgroup barriers. Only when more than 64 composites
// share d (long runs of equal keys) do further digits follow (select_threshold), and then a
// last pass takes every composite up to the threshold.
constexpr int kFirstDigitBits = 8;
template <typename Source, int NT>
__device__ void select_smallest(const Source &src, int r, int bits, int pos_bits, int32_t *out,
                                SelectShared<NT> &sh) {
    constexpr int kFirstBins = 1 << kFirstDigitBits;
    static_assert(NT >= kFirstBins && kFirstBins == 4 * 64, "four counts per lane of wavefront 0");
    const int digit = bits >= kFirstDigitBits ? kFirstDigitBits : bits;
    const int shift = bits - digit;
    if (threadIdx.x < kFirstBins) sh.hist[threadIdx.x] = 0;
    if (threadIdx.x == 0) {
        sh.n_out = 0;
        sh.n_tie = 0;
        // kept if fewer than r composites come (inputs that break their contract: a row's
        // counts short of its bound): a digit past every composite, so that all are taken and
        // nothing is written at or past out[r]
        sh.prefix = (uint64_t)kFirstBins << shift;
        sh.below = 0;
        sh.count = 0;
    }
    __syncthreads();
    src.for_each([&](uint64_t c) { atomicAdd(&sh.hist[(uint32_t)(c >> shift)], 1u); });
    __syncthreads();
    if (threadIdx.x < 64) {  // lane l: digits 4 l .. 4 l + 3, ascending
        uint32_t c4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c4[j] = sh.hist[4 * threadIdx.x + j];
        const int own = (int)(c4[0] + c4[1] + c4[2] + c4[3]);
        const int incl = wave_incl_scan(own);
        int before = incl - own;
        if (before < r && incl >= r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = (int)c4[j];
                if (before < r && before + c >= r) {
                    sh.prefix = (uint64_t)(4 * threadIdx.x + j) << shift;
                    sh.below = before;
                    sh.count = c;
                }
                before += c;
            }
        }
    }
    __syncthreads();
    const uint64_t top = sh.prefix;
    const uint64_t d = top >> shift;
    const int below = sh.below, cnt = sh.count;
    const bool whole = below + cnt == r;
    const uint64_t pos_mask = ((uint64_t)1 << pos_bits) - 1;
    if (!whole && cnt > 64) {
        const uint64_t threshold = select_threshold(src, r - below, bits, sh, top, digit);
        src.for_each([&](uint64_t c) {  // (n_out is still zero)
            const bool take = c <= threshold;  // the smaller digits too
            const uint32_t slot = wave_slot(take, &sh.n_out);
            if (take && slot < (uint32_t)r) out[slot] = (int32_t)(c & pos_mask);
        });
        return;
    }
    src.for_each([&](uint64_t c) {
        const uint64_t cd = c >> shift;
        const bool take = cd < d || (whole && cd == d);
        const uint32_t slot = wave_slot(take, &sh.n_out);
        if (take && slot < (uint32_t)r) out[slot] = (int32_t)(c & pos_mask);
        if (!whole) {
            const bool tie = cd == d;
            const uint32_t ts = wave_slot(tie, &sh.n_tie);
            if (tie && ts < 64u) sh.ties[ts] = c;
        }
    });
    if (whole) return;
    __syncthreads();  // the composites of digit d are in sh.ties
    if (threadIdx.x < 64) wave_select_out(sh.ties, cnt, r - below, shift, pos_bits, out + below);
}

template <int NT = kSelectThreads>
struct RowBin {  // every key of the row inside the threshold bin, read from the logits
    const float *x;
    int64_t n;
    uint32_t bin;
    int pos_bits;
    template <typename F>
    __device__ __forceinline__ void for_each(F &&f) const {
        for (int64_t i = threadIdx.x; i < n; i += NT) {
            const uint32_t u = order_key(x[i]);
            if ((u >> kBinShift) == bin) f(composite(u, (uint32_t)i, pos_bits));
        }
    }
};

}  // namespace dsaidx
