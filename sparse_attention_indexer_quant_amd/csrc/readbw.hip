// Bandwidth references, not steps of the indexer path: a plain read of paged key-cache
// sections (the bandwidth a kernel that only streams the scorer's pages reaches, against which
// the scorer is measured), and a plain contiguous read of a buffer (the device's read ceiling
// at a given size).
//
// It reads exactly the bytes score_paged reads from the cache -- the section of every block of
// every request below the request's key count -- with score_paged's grid (the same workgroups,
// wavefronts, pages per wavefront and request rotation) and the same per-lane loads (four
// 1 KB tiles of 16-B loads plus the 256 B of scale words for MXFP4; eight tiles for FP8), but
// no arithmetic: each lane XORs the words it loads and every wavefront writes one word, so the
// loads are kept.
#include "device_common.h"
#include "launch.h"

namespace dsaidx {

constexpr int kReadRing = 4;  // page buffers per wavefront: three pages' loads in flight

template <int TILES>
struct SectionRegs {
    uint4 v[TILES];
    uint32_t s;
};

template <int TILES>
__device__ __forceinline__ void load_section(SectionRegs<TILES> &r, const uint8_t *sec, uint32_t lane) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) r.v[t] = *reinterpret_cast<const uint4 *>(sec + t * 1024u + lane * 16u);
    r.s = *reinterpret_cast<const uint32_t *>(sec + TILES * 1024u + lane * 4u);
}

template <int TILES>
__device__ __forceinline__ uint32_t xor_section(const SectionRegs<TILES> &r) {
    uint32_t acc = r.s;
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc ^= r.v[t].x ^ r.v[t].y ^ r.v[t].z ^ r.v[t].w;
    return acc;
}

// Each wavefront streams its pages through a ring of kReadRing register buffers, as the scorer
// does: every load is issued unconditionally (a slot past the wavefront's pages, or a table
// entry that names no page, reads page 0 and is not counted), so the hardware wait before each
// page's XOR counts exactly and the loads of the next pages stay in flight.
template <int TILES>
__global__ __launch_bounds__(64 * kScoreWaves) void read_sections_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ seq_lens,
    int64_t max_blocks, int64_t num_requests, int pages_per_wave,
    const uint8_t *__restrict__ cache, int64_t page_stride, int64_t num_pages,
    uint32_t *__restrict__ out) {
    const uint32_t lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // workgroup b: chunk b / R of request (b + chunk) mod R, as in score_paged
    const uint32_t R = (uint32_t)num_requests;
    const uint32_t chunk = __builtin_amdgcn_readfirstlane(blockIdx.x / R);
    uint32_t req = blockIdx.x - chunk * R + chunk % R;
    if (req >= R) req -= R;
    const int PW = pages_per_wave;
    const int64_t blk_first = (int64_t)chunk * kScoreWaves * PW + wave;
    int64_t seq = seq_lens[req];
    seq = seq < 0 ? 0 : (seq > max_blocks * kPageTokens ? max_blocks * kPageTokens : seq);
    const int64_t nblk = (seq + kPageTokens - 1) / kPageTokens;
    // this wavefront's pages: blocks blk_first + 4 p below nblk, one table entry per lane
    const int64_t blk = blk_first + (int64_t)kScoreWaves * lane;
    const int bt_lane = (int)lane < PW && blk < nblk ? block_table[(int64_t)req * max_blocks + blk] : -1;
    int run = blk_first < nblk ? (int)((nblk - blk_first + kScoreWaves - 1) / kScoreWaves) : 0;
    run = run < PW ? run : PW;
    const uint32_t npages = num_pages < INT32_MAX ? (uint32_t)num_pages : (uint32_t)INT32_MAX;
    auto page = [&](int p) -> int {  // run page p's table entry, or -1
        const int pg = p < run ? __builtin_amdgcn_readlane(bt_lane, p) : -1;
        return (uint32_t)pg < npages ? pg : -1;
    };
    auto section = [&](int p) {
        const int pg = page(p);
        return cache + (int64_t)(pg >= 0 ? pg : 0) * page_stride;
    };
    SectionRegs<TILES> buf[kReadRing];
    uint32_t acc = 0;
#pragma unroll
    for (int p = 0; p < kReadRing - 1; ++p) load_section(buf[p], section(p), lane);
    for (int base = 0; base < run; base += kReadRing) {
#pragma unroll
        for (int slot = 0; slot < kReadRing; ++slot) {
            asm volatile("" ::: "memory");  // keep the ring as written (emits nothing)
            const int p = base + slot;
            load_section(buf[(slot + kReadRing - 1) % kReadRing], section(p + kReadRing - 1), lane);
            const uint32_t x = xor_section(buf[slot]);
            acc ^= page(p) >= 0 ? x : 0u;
        }
    }
    auto x = [](uint32_t a, uint32_t b) { return a ^ b; };
    acc = xor_combine<1>(acc, x);
    acc = xor_combine<2>(acc, x);
    acc = xor_combine<4>(acc, x);
    acc = xor_combine<8>(acc, x);
    acc = xor_combine<16>(acc, x);
    acc = xor_combine<32>(acc, x);
    if (lane == 0) out[(int64_t)blockIdx.x * kScoreWaves + wave] = acc;
}

// A contiguous read of n16 16-byte words: workgroup b takes words [b * 256 U, (b + 1) * 256 U)
// and then every gridDim.x * 256 U further; each lane issues its U loads (consecutive lanes on
// consecutive words) before it uses any, and every wavefront writes the XOR of what it read.
template <int U>
__global__ __launch_bounds__(256) void read_stream_kernel(const uint4 *__restrict__ buf, int64_t n16,
                                                          uint32_t *__restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * 256 * U;
    uint32_t acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + (int64_t)u * 256;
            v[u] = i < n16 ? buf[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    auto x = [](uint32_t a, uint32_t b) { return a ^ b; };
    acc = xor_combine<1>(acc, x);
    acc = xor_combine<2>(acc, x);
    acc = xor_combine<4>(acc, x);
    acc = xor_combine<8>(acc, x);
    acc = xor_combine<16>(acc, x);
    acc = xor_combine<32>(acc, x);
    if ((threadIdx.x & 63) == 0) out[(int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_read_stream(const void *buf, int64_t bytes, int workgroups, uint32_t *out,
                              hipStream_t stream) {
    hipLaunchKernelGGL(read_stream_kernel<8>, dim3((unsigned)workgroups), dim3(256), 0, stream,
                       static_cast<const uint4 *>(buf), bytes / 16, out);
    return hipGetLastError();
}

int64_t read_sections_words(int64_t num_requests, int64_t max_blocks) {
    return score_geometry(num_requests, max_blocks).chunks * num_requests * kScoreWaves;
}

hipError_t launch_read_sections(int fmt, const void *cache, int64_t num_pages, int64_t page_stride,
                                const int32_t *block_table, int64_t num_requests,
                                int64_t max_blocks, const int32_t *seq_lens, uint32_t *out,
                                hipStream_t stream) {
    const ScoreGeometry geo = score_geometry(num_requests, max_blocks);
    const dim3 grid((unsigned)(geo.chunks * num_requests)), block(64 * kScoreWaves);
    if (fmt == kFmtMxfp4)
        hipLaunchKernelGGL(read_sections_kernel<4>, grid, block, 0, stream, block_table, seq_lens,
                           max_blocks, num_requests, geo.pages_per_wave,
                           static_cast<const uint8_t *>(cache), page_stride, num_pages, out);
    else
        hipLaunchKernelGGL(read_sections_kernel<8>, grid, block, 0, stream, block_table, seq_lens,
                           max_blocks, num_requests, geo.pages_per_wave,
                           static_cast<const uint8_t *>(cache), page_stride, num_pages, out);
    return hipGetLastError();
}

}  // namespace dsaidx
