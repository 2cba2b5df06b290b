// Workspace layout shared by the top-k kernels and the scorer that can fill its histograms.
//
// The selection works on segments of a row's keys: a histogram of the top 12 order-key bits
// per (row, segment) and its 64-bin coarse sums, then per-row threshold state, per-segment output offsets and a
// candidate list per row. Either the standalone histogram kernel (segments of 4096..32768
// keys) or the scorer (segments = one scoring workgroup's run of pages) writes the
// histograms; the rest of the selection only needs the segment count and length.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

constexpr int kBins = 4096;              // top 12 order-key bits
constexpr int kBinShift = 20;
constexpr int kCoarseBins = 64;          // top 6 order-key bits: fine bins [64 c, 64 c + 64)
constexpr int kCandCap = 8192;           // candidate (key, position) pairs kept per row
constexpr int kMaxRowSegments = 1024;    // segments per row the threshold kernel handles

struct RowState {
    uint32_t bin;          // threshold bin
    int32_t above;         // keys above the threshold bin
    int32_t remaining;     // keys still to take from inside the bin
    uint32_t n_cand;       // keys inside the bin
};

struct TopkWorkspace {
    RowState *state;
    uint16_t *seghist;  // [rows][nseg][kBins]; a block of 64 is valid only where its coarse sum
                        // is nonzero (the scorer skips empty blocks)
    uint16_t *coarse;   // [rows][nseg][kCoarseBins]: sums of 64 consecutive fine bins
    uint2 *segoff;      // [rows][nseg]: first output slot, first candidate slot
    uint2 *cand;        // [rows][kCandCap]: order key, position
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline TopkWorkspace carve(void *ws, int64_t rows, int64_t nseg) {
    char *p = static_cast<char *>(ws);
    TopkWorkspace w;
    w.state = reinterpret_cast<RowState *>(p);
    p += align256(sizeof(RowState) * rows);
    w.seghist = reinterpret_cast<uint16_t *>(p);
    p += align256(sizeof(uint16_t) * kBins * nseg * rows);
    w.coarse = reinterpret_cast<uint16_t *>(p);
    p += align256(sizeof(uint16_t) * kCoarseBins * nseg * rows);
    w.segoff = reinterpret_cast<uint2 *>(p);
    p += align256(sizeof(uint2) * nseg * rows);
    w.cand = reinterpret_cast<uint2 *>(p);
    return w;
}

inline size_t topk_layout_bytes(int64_t rows, int64_t nseg) {
    return align256(sizeof(RowState) * rows) + align256(sizeof(uint16_t) * kBins * nseg * rows) +
           align256(sizeof(uint16_t) * kCoarseBins * nseg * rows) +
           align256(sizeof(uint2) * nseg * rows) + align256(sizeof(uint2) * (size_t)kCandCap * rows);
}

}  // namespace dsaidx
