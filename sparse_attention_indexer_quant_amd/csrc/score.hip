// Paged indexer scoring on gfx950 scaled MFMA.
//
// Page "vllm.models.kimi_k3.amd.ops.fp4_indexer", score_paged: one bounded query tile is
// scored against its requests' paged keys with shared-key row groups (all query rows of a
// request share each key load); cache sections are addressed through the physical page
// stride of merged caches; the head weights carry the model's head factors but not the
// FP4 block scales. Page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index",
// module text: the MX scales stay inside the logits contraction.
//
//   logit[r, p] = sum_h w[r, h] * max(0, q[r, h] . k[p])
//
// Contraction: v_mfma_scale_f32_16x16x128_f8f6f4, A = 16 heads x 128 of one query row,
// B = 128 x 16 key tokens. Operand lane l holds row/column (l % 16) and the 32-value K block
// (l / 16) -- exactly one MX block, so each lane's UE8M0 byte is its block scale. D lane l
// holds heads 4 * (l / 16) + i, i < 4, of token (l % 16). ReLU and the head weight are
// applied per lane, the head sum finishes with two cross-lane adds, and lane l ends up with
// the logit of token l of the page, so each row's 64 logits go out as one 256-byte store.
//
// FP8 keys take another route: the scaled MFMA sums each 32-value FP8 block with only about
// 13 bits below the block's largest product (448^2 + 1 comes out as 448^2), which cannot hold
// the 1e-5 logit tolerance once a head has outliers. E4M3 values are exactly representable in
// BF16, so the FP8 path widens both operands to BF16 in registers (v_cvt_pk_f32_fp8 plus a
// byte permute) and contracts on v_mfma_f32_16x16x32_bf16, whose sums kept every probed case
// exact. MXFP4 products span at most 2^7 (0.25 .. 36), so the FP4 MFMA is exact as it is.
//
// Work split: one workgroup of 4 wavefronts covers 4 * PPW consecutive pages of one request;
// each wavefront loads its PPW pages into registers first (all of them in flight at once),
// then runs the rows of the request over them in groups of RG rows.
#include "device_common.h"
#include "launch.h"

namespace dsaidx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;

__device__ __forceinline__ v4f mfma_fp4(const uint4 &a, const uint4 &b, int sa, int sb) {
    const v8i va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format selectors 4 = E2M1 for both operands; byte 0 of each scale register
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, zero, 4, 4, 0, sa, 0, sb);
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));

// Eight E4M3 bytes -> eight BF16 values (exact): the hardware FP8 -> FP32 conversion, then the
// high halves of two FP32 results packed into one dword.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    uint4 r;
    r.x = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
    r.y = __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u);
    r.z = __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u);
    r.w = __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), 0x07060302u);
    return r;
}

// The lane's 32 FP8 bytes (two uint4) as four 8-value BF16 K slices.
__device__ __forceinline__ void e4m3x32_to_bf16(const uint4 &x0, const uint4 &x1, uint4 out[4]) {
    out[0] = e4m3x8_to_bf16(x0.x, x0.y);
    out[1] = e4m3x8_to_bf16(x0.z, x0.w);
    out[2] = e4m3x8_to_bf16(x1.x, x1.y);
    out[3] = e4m3x8_to_bf16(x1.z, x1.w);
}

// One head's 128-value dot of 16 heads x 16 tokens as four K = 32 BF16 MFMAs. Lane group g
// holds columns [32 g, 32 g + 32) of its row / token; step kk takes 8 of them. A and B use
// the same split, so every column pairs with itself.
__device__ __forceinline__ v4f mfma_bf16_head(const uint4 qa[4], const uint4 kb[4]) {
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, qa[kk]),
                                                   __builtin_bit_cast(v8bf, kb[kk]), c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ float relu_dot4(const v4f &c, const float *w, float acc) {
    acc = fmaf(w[0], fmaxf(c[0], 0.f), acc);
    acc = fmaf(w[1], fmaxf(c[1], 0.f), acc);
    acc = fmaf(w[2], fmaxf(c[2], 0.f), acc);
    acc = fmaf(w[3], fmaxf(c[3], 0.f), acc);
    return acc;
}

// Sum the four lane groups (l / 16) of each tile's partials and leave tile t's token n in
// lane 16 t + n.
__device__ __forceinline__ float head_sum_to_token(float p0, float p1, float p2, float p3, int grp) {
    p0 += __shfl_xor(p0, 16);
    p1 += __shfl_xor(p1, 16);
    p2 += __shfl_xor(p2, 16);
    p3 += __shfl_xor(p3, 16);
    p0 += __shfl_xor(p0, 32);
    p1 += __shfl_xor(p1, 32);
    p2 += __shfl_xor(p2, 32);
    p3 += __shfl_xor(p3, 32);
    return grp == 0 ? p0 : grp == 1 ? p1 : grp == 2 ? p2 : p3;
}

template <int FMT, int H, int RG, int PPW>
__global__ __launch_bounds__(256) void score_paged_kernel(
    const uint8_t *__restrict__ q, int64_t q_row_stride, const uint16_t *__restrict__ w,
    int64_t w_row_stride, const uint8_t *__restrict__ cache, int64_t num_pages,
    int64_t page_stride, const int32_t *__restrict__ block_table, int64_t max_blocks,
    int64_t chunks, const int32_t *__restrict__ query_starts,
    const int32_t *__restrict__ row_ends, int64_t num_rows, int max_query_len,
    float *__restrict__ logits, int64_t logits_row_stride) {
    constexpr int HT = H / 16;  // 16-head tiles
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int l16 = lane & 15, grp = lane >> 4;
    const int64_t req = blockIdx.x / chunks;
    const int64_t chunk = blockIdx.x % chunks;
    const int64_t blk0 = (chunk * kWaves + wave) * PPW;
    const int64_t width = max_blocks * kPageTokens;

    int64_t r0 = query_starts[req], r1 = query_starts[req + 1];
    if (r0 < 0) return;
    if (r1 > r0 + max_query_len) r1 = r0 + max_query_len;
    if (r1 > num_rows) r1 = num_rows;
    const int nrows = (int)(r1 - r0);
    if (nrows <= 0) return;

    // Keys this request needs: the largest bound over its rows.
    int kmax = lane < nrows ? row_ends[r0 + lane] : 0;
    for (int m = 1; m < 64; m <<= 1) kmax = max(kmax, __shfl_xor(kmax, m));
    kmax = __builtin_amdgcn_readfirstlane(kmax);
    const int64_t kext = kmax < width ? kmax : width;
    if (blk0 * kPageTokens >= kext) return;

    // ---- stream this wavefront's pages into registers ----
    bool valid[PPW];
    uint4 kp[PPW][4][FMT == kFmtMxfp4 ? 1 : 2];
    uint32_t ks[PPW][4];  // MXFP4: UE8M0 byte of (token, block); FP8: FP32 scale bits of token
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
        const int64_t blk = blk0 + p;
        int page = -1;
        if (blk * kPageTokens < kext)
            page = __builtin_amdgcn_readfirstlane(block_table[req * max_blocks + blk]);
        valid[p] = page >= 0 && page < num_pages;
        if (valid[p]) {
            const uint8_t *sec = cache + (int64_t)page * page_stride;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int tok = t * 16 + l16;
                if constexpr (FMT == kFmtMxfp4) {
                    kp[p][t][0] = *reinterpret_cast<const uint4 *>(sec + tok * 64 + grp * 16);
                    ks[p][t] = *reinterpret_cast<const uint32_t *>(sec + 4096 + tok * 4) >> (8 * grp);
                } else {
                    const uint4 *src = reinterpret_cast<const uint4 *>(sec + tok * 128 + grp * 32);
                    kp[p][t][0] = src[0];
                    kp[p][t][1] = src[1];
                    ks[p][t] = *reinterpret_cast<const uint32_t *>(sec + 8192 + tok * 4);
                }
            }
        }
    }

    for (int rg = 0; rg < nrows; rg += RG) {
        // ---- query operands and head weights of RG rows ----
        uint4 qa[RG][HT][FMT == kFmtMxfp4 ? 1 : 4];
        int qs[RG][HT];
        float wt[RG][HT][4];
        int rend[RG];
#pragma unroll
        for (int j = 0; j < RG; ++j) {
            const int64_t row = r0 + rg + j;
            const bool active = rg + j < nrows;
            int e = active ? row_ends[row] : 0;
            e = __builtin_amdgcn_readfirstlane(e);
            rend[j] = (int64_t)e < width ? e : (int)width;
            const uint8_t *qrow = q + (active ? row : r0) * q_row_stride;
            const uint16_t *wrow = w + (active ? row : r0) * w_row_stride;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const int head = ht * 16 + l16;
                if constexpr (FMT == kFmtMxfp4) {
                    qa[j][ht][0] = *reinterpret_cast<const uint4 *>(qrow + head * 64 + grp * 16);
                    qs[j][ht] = qrow[H * 64 + head * 4 + grp];
                } else {
                    const uint4 *src = reinterpret_cast<const uint4 *>(qrow + head * 128 + grp * 32);
                    e4m3x32_to_bf16(src[0], src[1], qa[j][ht]);
                    qs[j][ht] = 0;
                }
                const uint2 wb = *reinterpret_cast<const uint2 *>(wrow + ht * 16 + grp * 4);
                wt[j][ht][0] = bf16_lo(wb.x);
                wt[j][ht][1] = bf16_hi(wb.x);
                wt[j][ht][2] = bf16_lo(wb.y);
                wt[j][ht][3] = bf16_hi(wb.y);
            }
        }

#pragma unroll
        for (int p = 0; p < PPW; ++p) {
            if (!valid[p]) continue;
            const int64_t kbase = (blk0 + p) * kPageTokens;
            float part[RG][4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                uint4 kb[FMT == kFmtMxfp4 ? 1 : 4];  // FP8: this tile's keys widened to BF16
                if constexpr (FMT == kFmtFp8) e4m3x32_to_bf16(kp[p][t][0], kp[p][t][1], kb);
#pragma unroll
                for (int j = 0; j < RG; ++j) {
                    float acc = 0.f;
                    if (rg + j < nrows && kbase < rend[j]) {
#pragma unroll
                        for (int ht = 0; ht < HT; ++ht) {
                            v4f c;
                            if constexpr (FMT == kFmtMxfp4)
                                c = mfma_fp4(qa[j][ht][0], kp[p][t][0], qs[j][ht], (int)ks[p][t]);
                            else
                                c = mfma_bf16_head(qa[j][ht], kb);
                            acc = relu_dot4(c, wt[j][ht], acc);
                        }
                        if constexpr (FMT == kFmtFp8) acc *= __uint_as_float(ks[p][t]);  // s_k > 0
                    }
                    part[j][t] = acc;
                }
            }
#pragma unroll
            for (int j = 0; j < RG; ++j) {
                if (rg + j >= nrows || kbase >= rend[j]) continue;
                const float out = head_sum_to_token(part[j][0], part[j][1], part[j][2], part[j][3], grp);
                const int64_t key = kbase + lane;
                if (key < rend[j]) logits[(r0 + rg + j) * logits_row_stride + key] = out;
            }
        }
    }
}

template <int FMT, int H, int RG>
static hipError_t launch_score_rg(const ScoreArgs &a, hipStream_t stream) {
    constexpr int PPW = FMT == kFmtMxfp4 ? 4 : 2;
    const int64_t pages_per_wg = (int64_t)kWaves * PPW;
    const int64_t chunks = (a.max_blocks + pages_per_wg - 1) / pages_per_wg;
    const dim3 grid((unsigned)(chunks * a.num_requests)), block(256);
    hipLaunchKernelGGL((score_paged_kernel<FMT, H, RG, PPW>), grid, block, 0, stream,
                       static_cast<const uint8_t *>(a.q), a.q_row_stride,
                       static_cast<const uint16_t *>(a.w), a.w_row_stride,
                       static_cast<const uint8_t *>(a.cache), a.num_pages, a.page_stride,
                       a.block_table, a.max_blocks, chunks, a.query_starts, a.row_ends,
                       a.num_rows, a.max_query_len, a.logits, a.logits_row_stride);
    return hipGetLastError();
}

template <int FMT, int H>
static hipError_t launch_score_h(const ScoreArgs &a, hipStream_t stream) {
    if (a.max_query_len <= 1) return launch_score_rg<FMT, H, 1>(a, stream);
    if constexpr (FMT == kFmtFp8) {
        // FP8 queries occupy 4x the registers once widened to BF16: at most 2 rows per group
        return launch_score_rg<FMT, H, 2>(a, stream);
    } else {
        if (a.max_query_len <= 2) return launch_score_rg<FMT, H, 2>(a, stream);
        return launch_score_rg<FMT, H, 4>(a, stream);
    }
}

template <int FMT>
static hipError_t launch_score_fmt(const ScoreArgs &a, hipStream_t stream) {
    switch (a.heads) {
        case 16: return launch_score_h<FMT, 16>(a, stream);
        case 32: return launch_score_h<FMT, 32>(a, stream);
        default: return launch_score_h<FMT, 64>(a, stream);
    }
}

hipError_t launch_score_paged(const ScoreArgs &a, hipStream_t stream) {
    return a.fmt == kFmtMxfp4 ? launch_score_fmt<kFmtMxfp4>(a, stream)
                              : launch_score_fmt<kFmtFp8>(a, stream);
}

}  // namespace dsaidx
