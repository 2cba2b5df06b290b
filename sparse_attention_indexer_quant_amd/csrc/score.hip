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
// applied per lane, the head sum finishes with three cross-row swaps, and lane l ends up
// with the logit of token l of the page, so each row's 64 logits go out as one 256-B store.
//
// FP8 keys (scale stored as FP32, or with mx as its UE8M0 exponent byte; the scale is a power
// of two either way) take another route: the scaled MFMA sums each 32-value FP8 block with only about
// 13 bits below the block's largest product (448^2 + 1 comes out as 448^2), which cannot hold
// the 1e-5 logit tolerance once a head has outliers. E4M3 values are exactly representable in
// BF16, so the FP8 path widens both operands to BF16 in registers (v_cvt_pk_f32_fp8 plus a
// byte permute) and contracts on v_mfma_f32_16x16x32_bf16, whose sums kept every probed case
// exact. MXFP4 products span at most 2^7 (0.25 .. 36), so the FP4 MFMA is exact as it is.
//
// Work split: a workgroup's 4 wavefronts each stream a run of consecutive pages of one
// request through a ring of page buffers, for all rows of the request (in groups of RG
// rows held in registers).
//
// With HIST, the kernel also feeds the top-k selection: each workgroup counts its logits per
// row into an LDS histogram of the top 12 order-key bits (two 16-bit counts per word) and
// writes it as the (row, segment) histogram of a top-k workspace, segment = the workgroup's
// run of keys. The selection then skips its own pass over the logits.
//
// With FUSED (index_score_hist), the kernel also makes the step's inputs (page
// "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index", DsaIndex; page
// "vllm.models.kimi_k3.amd.ops.fp4_indexer", decode_layout): the MXFP4 query operands, the
// head weights, the new keys' LayerNorm, quantization and insert, and the row layout.
#include <type_traits>

#include "device_common.h"
#include "key_norm.h"
#include "launch.h"
#include "select.h"
#include "topk_layout.h"

namespace dsaidx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = kScoreWaves;
// the histogram flush gives each lane of the workgroup 16 consecutive fine bins
static_assert(64 * kWaves * 16 == kBins, "one flush lane per 16 fine bins");
constexpr int kMaxPagesPerWave = 16;

// A's scale is byte 0 of `sa`; B's is byte T of `sb` (T = the key tile: the page's scale
// dword holds one byte per tile, see tile_scales)
template <int T>
__device__ __forceinline__ v4f mfma_fp4(const uint4 &a, const uint4 &b, int sa, int sb) {
    const v8i va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format selectors 4 = E2M1 for both operands
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, zero, 4, 4, 0, sa, T, sb);
}

__device__ __forceinline__ v4f mfma_fp4_tile(const uint4 &a, const uint4 &b, int sa, int sb, int t) {
    switch (t) {  // t is a constant after unrolling
        case 0: return mfma_fp4<0>(a, b, sa, sb);
        case 1: return mfma_fp4<1>(a, b, sa, sb);
        case 2: return mfma_fp4<2>(a, b, sa, sb);
        default: return mfma_fp4<3>(a, b, sa, sb);
    }
}

// A page's 256 UE8M0 bytes are loaded as one dword per lane: lane L holds the four block
// scales of token L. The MFMA wants, in lane (l16, grp) for tile t, the scale of token
// 16 t + l16, block grp: byte grp of lane (t, l16). That is a 4 x 4 byte transpose over the
// four lane rows, done as two exchanges: rows r and r ^ 2 swap 16-bit halves, then rows r
// and r ^ 1 swap bytes. `sel32` / `sel16` are the lane's byte selectors of the two steps.
__device__ __forceinline__ uint32_t tile_scales(uint32_t raw, uint32_t sel32, uint32_t sel16) {
    const auto a = __builtin_amdgcn_permlane32_swap(raw, raw, false, false);
    const uint32_t y = __builtin_amdgcn_perm(a[1], a[0], sel32);
    const auto b = __builtin_amdgcn_permlane16_swap(y, y, false, false);
    return __builtin_amdgcn_perm(b[1], b[0], sel16);
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

// max(0, x) on the bit pattern: non-negative floats compare as non-negative integers, and
// negative floats (and -0) have the sign bit set, so an integer max with 0 returns +0 for
// them. One integer max, and no NaN canonicalization.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// acc + sum_i w_i * max(0, c_i) for the lane's 4 heads; w holds 4 BF16 weights.
__device__ __forceinline__ float relu_dot4(const v4f &c, const uint2 &w, float acc) {
    acc = fmaf(bf16_lo(w.x), relu(c[0]), acc);
    acc = fmaf(bf16_hi(w.x), relu(c[1]), acc);
    acc = fmaf(bf16_lo(w.y), relu(c[2]), acc);
    acc = fmaf(bf16_hi(w.y), relu(c[3]), acc);
    return acc;
}

// The same sum with the weights already in FP32, in the same order.
__device__ __forceinline__ float relu_dot4(const v4f &c, const float4 &w, float acc) {
    acc = fmaf(w.x, relu(c[0]), acc);
    acc = fmaf(w.y, relu(c[1]), acc);
    acc = fmaf(w.z, relu(c[2]), acc);
    acc = fmaf(w.w, relu(c[3]), acc);
    return acc;
}

// 4 BF16-valued floats back to the packed BF16 pair layout of the registers (exact: their
// low 16 bits are zero).
__device__ __forceinline__ uint2 bf16_pair_bits(const float4 &w) {
    return make_uint2((__float_as_uint(w.x) >> 16) | (__float_as_uint(w.y) & 0xFFFF0000u),
                      (__float_as_uint(w.z) >> 16) | (__float_as_uint(w.w) & 0xFFFF0000u));
}

// Head sum across the four lane groups (rows of 16 lanes) for the page's four token tiles,
// leaving tile t's token n in lane 16 t + n; p_t holds each lane's partial for tile t.
// A reduce-scatter on the cross-row swap instructions: swapping halves pairs tiles (0, 2)
// and (1, 3) so the lower half keeps tiles 0 / 1 and the upper half tiles 2 / 3, then
// swapping odd and even rows finishes each tile in its own row. Three swaps, three adds.
__device__ __forceinline__ float head_sum_to_token(float p0, float p1, float p2, float p3) {
    const auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
    const float a = __uint_as_float(s02[0]) + __uint_as_float(s02[1]);  // rows 0,1: tile 0; rows 2,3: tile 2
    const float b = __uint_as_float(s13[0]) + __uint_as_float(s13[1]);  // rows 0,1: tile 1; rows 2,3: tile 3
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One page of keys held in registers: per lane, tile t (tokens 16t .. 16t+15) contributes
// its token (l % 16), 32-value block (l / 16): 16 B for MXFP4 (plus that block's UE8M0 byte),
// 32 B for FP8 (plus the token's FP32 scale).
template <int FMT>
struct PageRegs {
    uint4 kp[4][FMT == kFmtMxfp4 ? 1 : 2];
    // MXFP4: the four block scales of token `lane` (as loaded; tile_scales rearranges them);
    // FP8: per tile, the token's 32-bit scale
    uint32_t ks[FMT == kFmtMxfp4 ? 1 : 4];
};

// Loads one page section into registers. The caller always issues the loads (a page that
// is not scored reads a valid stand-in page instead), so the instruction stream has no
// conditional loads and every wait can count exactly. Each load addresses as (uniform base
// in scalar registers: section + tile offset) + (the lane's unsigned 32-bit offset), which
// keeps the address arithmetic off the vector ALUs.
template <int FMT>
struct LaneOffsets {
    uint32_t key;    // the lane's token row (l % 16) and K block (l / 16) within a tile
    uint32_t scale;  // the lane's scale byte (MXFP4) or its token's FP32 scale (FP8)
    __device__ __forceinline__ LaneOffsets(uint32_t l16, uint32_t grp)
        : key(FMT == kFmtMxfp4 ? l16 * 64u + grp * 16u : l16 * 128u + grp * 32u),
          scale(FMT == kFmtMxfp4 ? 4096u + (grp * 16u + l16) * 4u : 8192u + l16 * 4u) {}
};

template <int FMT>
__device__ __forceinline__ void load_page(PageRegs<FMT> &pg, const uint8_t *sec,
                                          const LaneOffsets<FMT> &off) {
#pragma unroll
    for (uint32_t t = 0; t < 4; ++t) {
        if constexpr (FMT == kFmtMxfp4) {
            const uint8_t *tile = sec + t * 1024u;         // 16 tokens x 64 B
            pg.kp[t][0] = *reinterpret_cast<const uint4 *>(tile + off.key);
            // token `lane`'s four UE8M0 bytes (one load for the page's 256 scale bytes)
            if (t == 0) pg.ks[0] = *reinterpret_cast<const uint32_t *>(sec + off.scale);
        } else {
            const uint8_t *tile = sec + t * 2048u;         // 16 tokens x 128 B
            pg.kp[t][0] = *reinterpret_cast<const uint4 *>(tile + off.key);
            pg.kp[t][1] = *reinterpret_cast<const uint4 *>(tile + off.key + 16u);
            pg.ks[t] = *reinterpret_cast<const uint32_t *>((sec + t * 64u) + off.scale);
        }
    }
}

template <int FMT, int H, int RG>
struct StepQueryLds {
    static constexpr int kTiles = RG * (H / 16);
    static constexpr int kParts = FMT == kFmtMxfp4 ? 1 : 4;  // FP8: 32 values widened to BF16
    uint4 qa[kTiles][kParts][64];
    // the lane's 4 head weights, BF16 values held as FP32 (exact), so that a page's weighted
    // head sum reads them ready to use instead of widening them on every page
    float4 wt[kTiles][64];
    int qs[kTiles][FMT == kFmtMxfp4 ? 64 : 1];
};

// Query operands, head weights and key bounds of one group of RG rows. With OPS_IN_LDS (the
// fused step inputs of four-row MXFP4 and two-row FP8 groups) the operands stay in the
// workgroup's LDS tiles and each page reads them there: holding them in registers took a
// four-row MXFP4 group to about 200 VGPRs (two wavefronts per SIMD) and a two-row FP8 group,
// whose operands are widened to BF16, past the 256 VGPRs into AGPRs.
template <int FMT, int H, int RG, bool OPS_IN_LDS = false>
struct RowGroup {
    static constexpr int HT = H / 16;
    static constexpr int RR = OPS_IN_LDS ? 1 : RG;  // rows held in registers
    uint4 qa[RR][HT][FMT == kFmtMxfp4 ? 1 : 4];
    int qs[RR][HT];
    uint2 wt[RR][HT];  // 4 BF16 head weights, widened at use
    const StepQueryLds<FMT, H, RG> *ops = nullptr;
    int ops_lane = 0;
    int rend[RG];

    __device__ __forceinline__ uint4 qa_at(int j, int ht, int part = 0) const {
        if constexpr (OPS_IN_LDS) return ops->qa[j * HT + ht][part][ops_lane];
        else return qa[j][ht][part];
    }
    __device__ __forceinline__ int qs_at(int j, int ht) const {
        if constexpr (OPS_IN_LDS) return ops->qs[j * HT + ht][ops_lane];
        else return qs[j][ht];
    }
    // OPS_IN_LDS: 4 FP32 weights from the LDS tile; else 4 BF16 weights from registers
    __device__ __forceinline__ auto wt_at(int j, int ht) const {
        if constexpr (OPS_IN_LDS) return ops->wt[j * HT + ht][ops_lane];
        else return wt[j][ht];
    }

    __device__ __forceinline__ void load(const uint8_t *q, int64_t q_row_stride, const uint16_t *w,
                                         int64_t w_row_stride, const int32_t *row_ends,
                                         int64_t first, int64_t last, int64_t width, int l16,
                                         int grp) {
#pragma unroll
        for (int j = 0; j < RG; ++j) {
            const int64_t row = first + j;
            const bool active = row < last;
            int e = active ? row_ends[row] : 0;
            e = __builtin_amdgcn_readfirstlane(e);
            rend[j] = (int64_t)e < width ? e : (int)width;
            const uint8_t *qrow = q + (active ? row : first) * q_row_stride;
            const uint16_t *wrow = w + (active ? row : first) * w_row_stride;
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
                wt[j][ht] = *reinterpret_cast<const uint2 *>(wrow + ht * 16 + grp * 4);
            }
        }
    }

    // The operands made in the workgroup (StepQuery below), and bounds from the request's
    // sequence length: row r0 + i ends at max(0, seq - qlen + i + 1).
    template <typename Lds>
    __device__ __forceinline__ void from_lds(const Lds &s, int64_t r0, int seq, int qlen,
                                             int64_t first, int64_t last, int64_t width,
                                             int lane) {
        ops = &s;
        ops_lane = lane;
#pragma unroll
        for (int j = 0; j < RG; ++j) {
            const int64_t row = first + j;
            int64_t e = (int64_t)seq - qlen + (row - r0) + 1;
            e = e < 0 ? 0 : (e < width ? e : width);
            rend[j] = row < last ? (int)e : 0;
            if constexpr (!OPS_IN_LDS) {
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
#pragma unroll
                    for (int k = 0; k < (FMT == kFmtMxfp4 ? 1 : 4); ++k)
                        qa[j][ht][k] = s.qa[j * HT + ht][k][lane];
                    qs[j][ht] = FMT == kFmtMxfp4 ? s.qs[j * HT + ht][lane] : 0;
                    wt[j][ht] = bf16_pair_bits(s.wt[j * HT + ht][lane]);
                }
            }
        }
    }

    // Logits of one page for the group's rows. Rows past `count` are not computed: row 0, then
    // rows 1, 2 and 3 each only if present (one uniform branch each).
    __device__ __forceinline__ void score(const PageRegs<FMT> &pg, int kbase, int count,
                                          float *logits, int64_t first_row,
                                          int64_t logits_row_stride, int lane, int grp,
                                          uint32_t *hist, uint32_t sel32, uint32_t sel16,
                                          float *keep = nullptr) const {
        const uint32_t ksw = FMT == kFmtMxfp4 ? tile_scales(pg.ks[0], sel32, sel16) : 0u;
        score_rows<0, 1>(pg, ksw, kbase, count, logits, first_row, logits_row_stride, lane, grp,
                         hist, keep);
        if constexpr (RG > 1) {
            if (count > 1)
                score_rows<1, 2>(pg, ksw, kbase, count, logits, first_row, logits_row_stride,
                                 lane, grp, hist);
        }
        if constexpr (RG > 2) {
            if (count > 2)
                score_rows<2, 3>(pg, ksw, kbase, count, logits, first_row, logits_row_stride,
                                 lane, grp, hist);
        }
        if constexpr (RG > 3) {
            if (count > 3)
                score_rows<3, RG>(pg, ksw, kbase, count, logits, first_row, logits_row_stride,
                                  lane, grp, hist);
        }
    }

    // Rows [J0, J1) of the group. Each tile's (J1 - J0) x HT contractions are issued back to
    // back into separate results before any is read, so the matrix unit pipelines them instead
    // of waiting on each result in turn.
    template <int J0, int J1>
    __device__ __forceinline__ void score_rows(const PageRegs<FMT> &pg, uint32_t ksw, int kbase,
                                               int count,
                                               float *logits, int64_t first_row,
                                               int64_t logits_row_stride, int lane, int grp,
                                               uint32_t *hist, float *keep = nullptr) const {
        float part[RG][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint4 kb[FMT == kFmtMxfp4 ? 1 : 4];  // FP8: this tile's keys widened to BF16
            if constexpr (is_fp8(FMT)) e4m3x32_to_bf16(pg.kp[t][0], pg.kp[t][1], kb);
            v4f c[RG][HT];
#pragma unroll
            for (int j = J0; j < J1; ++j) {
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
                    if constexpr (FMT == kFmtMxfp4)
                        c[j][ht] = mfma_fp4_tile(qa_at(j, ht), pg.kp[t][0], qs_at(j, ht), (int)ksw, t);
                    else {
                        const uint4 q4[4] = {qa_at(j, ht, 0), qa_at(j, ht, 1), qa_at(j, ht, 2),
                                             qa_at(j, ht, 3)};
                        c[j][ht] = mfma_bf16_head(q4, kb);
                    }
                }
            }
#pragma unroll
            for (int j = J0; j < J1; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) acc = relu_dot4(c[j][ht], wt_at(j, ht), acc);
                // the token's scale s_k > 0 (a power of two): FP32, or its UE8M0 exponent byte
                if constexpr (FMT == kFmtFp8) acc *= __uint_as_float(pg.ks[t]);
                if constexpr (FMT == kFmtFp8Mx) acc *= __uint_as_float((pg.ks[t] & 0xFFu) << 23);
                part[j][t] = acc;
            }
        }
#pragma unroll
        for (int j = J0; j < J1; ++j) {
            if (j >= count || kbase >= rend[j]) continue;
            const float out = head_sum_to_token(part[j][0], part[j][1], part[j][2], part[j][3]);
            float *row = logits + (first_row + j) * logits_row_stride + kbase;
            if (kbase + lane < rend[j]) {
                row[lane] = out;
                if (j == 0 && keep) keep[kbase + lane] = out;  // at the key's position
                if (hist) {
                    const uint32_t bin = order_key(out) >> kBinShift;
                    atomicAdd(&hist[j * (kBins / 2) + (bin >> 1)], 1u << (16 * (bin & 1)));
                }
            }
        }
    }
};

// The scorer's own MXFP4 query operands (fused step inputs), made with the step-input kernel's
// arithmetic so that they are bit-identical to the bytes it writes. A row group's RG x H/16
// operand tiles (row j, heads 16 ht .. 16 ht + 15) are dealt out over the workgroup's four
// wavefronts; lane (l16, grp) of a tile encodes the 32-value block grp of head 16 ht + l16
// -- the UE8M0 exponent of the block's largest magnitude, then the E2M1 codes of the values
// times 2^-e -- and rounds its four head weights times c_h to BF16. The tiles meet in the LDS
// in the lane layout of RowGroup's registers.
template <int FMT, int H, int RG>
struct StepQuery {
    static constexpr int HT = H / 16, kTiles = RG * HT, kPer = (kTiles + kWaves - 1) / kWaves;
    uint4 raw[kPer][4];
    uint32_t wraw[kPer][4];  // 32-bit: 16-bit lanes would be packed in pairs, which waits for the loads

    // Every load is issued, with no branch around it (a tile past the group reads tile 0's
    // rows), so that the wait for them leaves the page loads issued after them in flight.
    __device__ __forceinline__ void load(const uint16_t *q, int64_t q_row_stride,
                                         int64_t q_head_stride, const uint16_t *w_in,
                                         int64_t proj_row_stride, int64_t first, int64_t last,
                                         int wave, int l16, int grp) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            int it = wave + kWaves * m;
            if (it >= kTiles) it = 0;
            const int j = it / HT, ht = it % HT;
            const int64_t rr = first + j < last ? first + j : first;
            const uint4 *src = reinterpret_cast<const uint4 *>(
                q + rr * q_row_stride + (int64_t)(ht * 16 + l16) * q_head_stride + grp * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) raw[m][i] = src[i];
            const uint16_t *wrow = w_in + rr * proj_row_stride + ht * 16 + grp * 4;
#pragma unroll
            for (int i = 0; i < 4; ++i) wraw[m][i] = wrow[i];
        }
    }

    __device__ __forceinline__ void encode(StepQueryLds<FMT, H, RG> &s, float c_h, int wave,
                                           int lane) const {
        if constexpr (FMT != kFmtMxfp4) {
            encode_fp8(s, c_h, wave, lane);
            return;
        }
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int it = wave + kWaves * m;
            if (it >= kTiles) continue;
            float amax = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wd[4] = {raw[m][i].x, raw[m][i].y, raw[m][i].z, raw[m][i].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(wd[c])), fabsf(bf16_hi(wd[c]))));
            }
            const int ex = ue8m0_exponent(amax);
            uint32_t out[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t word = 0;
                word = e2m1_bf16_pair<0>(word, raw[m][i].x, ex);
                word = e2m1_bf16_pair<1>(word, raw[m][i].y, ex);
                word = e2m1_bf16_pair<2>(word, raw[m][i].z, ex);
                word = e2m1_bf16_pair<3>(word, raw[m][i].w, ex);
                out[i] = word;
            }
            uint32_t wb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wb[i] = bf16_bits_rne(__fmul_rn(bf16_val((uint16_t)wraw[m][i]), c_h));
            s.qa[it][0][lane] = make_uint4(out[0], out[1], out[2], out[3]);
            s.qs[it][lane] = ex + 127;
            s.wt[it][lane] = make_float4(__uint_as_float(wb[0] << 16), __uint_as_float(wb[1] << 16),
                                         __uint_as_float(wb[2] << 16), __uint_as_float(wb[3] << 16));
        }
    }

    // FP8 (the separate quantizer's arithmetic): per head, s = pow2_ceil(max(1e-10, amax) / 448)
    // over its 128 values -- the four lanes (l16, 0..3) of a head hold its four 32-value blocks
    // -- the E4M3 codes of v / s, widened exactly to BF16 for the MFMA, and the head weights
    // BF16(w * s * c_h); lane (l16, grp) weighs heads 4 grp + i, whose scales it takes from
    // lanes 4 grp + i.
    __device__ __forceinline__ void encode_fp8(StepQueryLds<FMT, H, RG> &s, float c_h, int wave,
                                               int lane) const {
        auto mx = [](float a, float b) { return fmaxf(a, b); };
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const int it = wave + kWaves * m;
            if (it >= kTiles) continue;
            float amax = 1e-10f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wd[4] = {raw[m][i].x, raw[m][i].y, raw[m][i].z, raw[m][i].w};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(wd[c])), fabsf(bf16_hi(wd[c]))));
            }
            amax = xor_combine<16>(amax, mx);
            amax = xor_combine<32>(amax, mx);
            const float sc = pow2_ceil(__fdiv_rn(amax, 448.0f));
            const float inv = __fdiv_rn(1.0f, sc);
            uint32_t codes[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t wd[4] = {raw[m][i].x, raw[m][i].y, raw[m][i].z, raw[m][i].w};
                const uint32_t lo = e4m3x4(__fmul_rn(bf16_lo(wd[0]), inv), __fmul_rn(bf16_hi(wd[0]), inv),
                                           __fmul_rn(bf16_lo(wd[1]), inv), __fmul_rn(bf16_hi(wd[1]), inv));
                const uint32_t hi = e4m3x4(__fmul_rn(bf16_lo(wd[2]), inv), __fmul_rn(bf16_hi(wd[2]), inv),
                                           __fmul_rn(bf16_lo(wd[3]), inv), __fmul_rn(bf16_hi(wd[3]), inv));
                codes[2 * i] = lo;
                codes[2 * i + 1] = hi;
            }
            uint4 widened[4];
            e4m3x32_to_bf16(make_uint4(codes[0], codes[1], codes[2], codes[3]),
                            make_uint4(codes[4], codes[5], codes[6], codes[7]), widened);
#pragma unroll
            for (int k = 0; k < 4; ++k) s.qa[it][k][lane] = widened[k];
            const int grp = lane >> 4;
            uint32_t wb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float si = __shfl(sc, 4 * grp + i);  // head 4 grp + i of the tile
                wb[i] = bf16_bits_rne(__fmul_rn(__fmul_rn(bf16_val((uint16_t)wraw[m][i]), si), c_h));
            }
            s.wt[it][lane] = make_float4(__uint_as_float(wb[0] << 16), __uint_as_float(wb[1] << 16),
                                         __uint_as_float(wb[2] << 16), __uint_as_float(wb[3] << 16));
        }
    }
};

// A new key in the page registers of the wavefront that scores its page: lane (l16, grp) of
// tile o / 16 with l16 = o % 16 takes the key's 16 payload bytes of block grp and its UE8M0
// byte from the staged key (64 payload bytes, then the 4 scale bytes).
__device__ __forceinline__ void patch_key(PageRegs<kFmtMxfp4> &pg, const uint8_t *staged, int o,
                                          int l16, int grp) {
    const uint4 v = *reinterpret_cast<const uint4 *>(staged + grp * 16);
    const uint32_t sc = *reinterpret_cast<const uint32_t *>(staged + 64);
    const bool mine = l16 == (o & 15);
    const uint32_t ms = grp * 16 + l16 == o ? 0xFFFFFFFFu : 0u;  // lane o holds token o's scales
    pg.ks[0] = (sc & ms) | (pg.ks[0] & ~ms);
    // bit masks in every tile: a branch or a select over the registers' values gets folded
    // into one access at a computed tile index or address, which puts them in scratch memory
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t m = mine && t == (o >> 4) ? 0xFFFFFFFFu : 0u;
        uint4 &k = pg.kp[t][0];
        k = make_uint4((v.x & m) | (k.x & ~m), (v.y & m) | (k.y & ~m), (v.z & m) | (k.z & ~m),
                       (v.w & m) | (k.w & ~m));
    }
}

// The FP8 form: lane (l16, grp) of tile o / 16 with l16 = o % 16 takes the key's 32 code bytes
// of block grp, and every lane of that token its scale word (staged: 128 code bytes, then the
// 4-byte scale word).
__device__ __forceinline__ void patch_key(PageRegs<kFmtFp8> &pg, const uint8_t *staged, int o,
                                          int l16, int grp) {
    const uint4 v0 = *reinterpret_cast<const uint4 *>(staged + grp * 32);
    const uint4 v1 = *reinterpret_cast<const uint4 *>(staged + grp * 32 + 16);
    const uint32_t sc = *reinterpret_cast<const uint32_t *>(staged + 128);
    const bool mine = l16 == (o & 15);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t m = mine && t == (o >> 4) ? 0xFFFFFFFFu : 0u;
        uint4 &a = pg.kp[t][0];
        uint4 &b = pg.kp[t][1];
        a = make_uint4((v0.x & m) | (a.x & ~m), (v0.y & m) | (a.y & ~m), (v0.z & m) | (a.z & ~m),
                       (v0.w & m) | (a.w & ~m));
        b = make_uint4((v1.x & m) | (b.x & ~m), (v1.y & m) | (b.y & ~m), (v1.z & m) | (b.z & ~m),
                       (v1.w & m) | (b.w & ~m));
        pg.ks[t] = (sc & m) | (pg.ks[t] & ~m);
    }
}
__device__ __forceinline__ void patch_key(PageRegs<kFmtFp8Mx> &pg, const uint8_t *staged, int o,
                                          int l16, int grp) {
    patch_key(reinterpret_cast<PageRegs<kFmtFp8> &>(pg), staged, o, l16, grp);
}

// Rows of request `req` from the query lengths: the first is the sum of the lengths before it
// (a wavefront sum, uniform), the count its own length. The first 256 lengths (four per lane)
// are loaded without conditions, at indices clamped into [0, R) (all in bounds), so a kernel
// can issue them early and later loads' waits count exactly; lengths beyond are summed in a
// loop of their own (requests past the 256th only).
struct FirstRowLoads {
    int v[4];
};

__device__ __forceinline__ FirstRowLoads issue_first_row(const int32_t *lens, int64_t R, int lane) {
    FirstRowLoads f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int64_t i = 64 * u + lane;
        f.v[u] = lens[i < R ? i : R - 1];
    }
    return f;
}

__device__ __forceinline__ int64_t finish_first_row(const FirstRowLoads &f, const int32_t *lens,
                                                    int64_t req, int lane) {
    int acc = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) acc += 64 * u + lane < req ? f.v[u] : 0;
    for (int64_t base = 256; base < req; base += 256) {
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = base + 64 * u + lane;
            v[u] = i < req ? lens[i] : 0;
        }
        acc += (v[0] + v[1]) + (v[2] + v[3]);
    }
    auto add = [](int a, int b) { return a + b; };
    acc = xor_combine<1>(acc, add);
    acc = xor_combine<2>(acc, add);
    acc = xor_combine<4>(acc, add);
    acc = xor_combine<8>(acc, add);
    acc = xor_combine<16>(acc, add);
    acc = xor_combine<32>(acc, add);
    return __builtin_amdgcn_readfirstlane(acc);
}

// Value of request slot q (q < 256) of a per-lane array holding request 64 u + lane in a[u].
__device__ __forceinline__ int request_value(const int (&a)[4], uint32_t q) {
    const uint32_t u = q >> 6;
    const int v = u == 0 ? a[0] : u == 1 ? a[1] : u == 2 ? a[2] : a[3];
    return __builtin_amdgcn_readlane(v, (int)(q & 63u));
}

// Work item of workgroup b in a longest-first order, for launches whose requests have different
// row counts (multi-row groups): request q holds nch[q] chunks of keys, each costing about its
// row count lvl[q] (1..4) times its pages; items run by level, most rows first, then by chunk,
// then by request (consecutive workgroups, on consecutive XCDs, take different requests). The
// hardware starts workgroups in index order, so the heaviest items start first and the light
// ones fill the machine at the end, instead of four-row chunks starting last and finishing
// long after the rest. A workgroup past every item gets chunk == chunks (nothing to score).
// Inputs per lane: request 64 u + lane in slot u (R <= 256 requests); output uniform.
struct WorkItem {
    uint32_t req, chunk;
};
__device__ __forceinline__ WorkItem longest_first_item(uint32_t b, const int (&lvl)[4],
                                                       const int (&nch)[4], uint32_t chunks) {
    auto add = [](int a, int c) { return a + c; };
    int level = 0;
    for (int L = 4; L >= 1 && level == 0; --L) {
        int t = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) t += lvl[u] == L ? nch[u] : 0;
        t = xor_combine<1>(t, add);
        t = xor_combine<2>(t, add);
        t = xor_combine<4>(t, add);
        t = xor_combine<8>(t, add);
        t = xor_combine<16>(t, add);
        t = xor_combine<32>(t, add);
        const uint32_t tot = (uint32_t)__builtin_amdgcn_readfirstlane(t);
        if (b < tot) level = L;
        else b -= tot;
    }
    if (level == 0) return {0u, chunks};
    for (uint32_t c = 0; c < chunks; ++c) {
        uint64_t m[4];
        uint32_t n = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            m[u] = __ballot(lvl[u] == level && (uint32_t)nch[u] > c);
            n += (uint32_t)__builtin_popcountll(m[u]);
        }
        if (b < n) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t k = (uint32_t)__builtin_popcountll(m[u]);
                if (b < k) {
                    uint64_t mm = m[u];
                    for (uint32_t i = 0; i < b; ++i) mm &= mm - 1;
                    return {64u * u + (uint32_t)__builtin_ctzll(mm), c};
                }
                b -= k;
            }
        }
        b -= n;
    }
    return {0u, chunks};
}

// a staged new key: MXFP4 64 payload + 4 scale bytes, FP8 128 code bytes + the scale word,
// padded to 16
template <int FMT>
constexpr int staged_key_bytes() { return FMT == kFmtMxfp4 ? 80 : 144; }

// Grid: requests x chunks; a workgroup's chunk is 4 PW consecutive pages of the request, which
// its 4 wavefronts take in turn (PW pages each). Workgroups map to (request, chunk) items
// chunk-major, or, for multi-row groups, longest first (longest_first_item). Each wavefront streams its pages through a
// ring of NB page buffers: the next NB - 1 pages' loads are in flight while one page is
// scored. Every prefetch is issued unconditionally (a page that is not scored reads page 0
// instead), so the loop carries the same loads across its back edge on every path and the
// hardware wait counts stay exact; conditional prefetches made the compiler wait for all loads
// there. The first NB - 1 page loads go out right after the query and row-bound loads. The
// arguments the first loads need come first: the library is built to preload the leading
// kernel arguments into scalar registers at wave launch.
//
// FUSED (with histograms, one row group per request: up to 4 rows for MXFP4, 2 for FP8 and
// FP8 "mx"): the step's inputs are made here
// instead of read -- `query_starts` holds the query lengths and `q` the BF16 query -- and the
// result equals the step-input kernel with decode_layout followed by the plain launch, with
// each row's new key at position seq - qlen + i of its request (the slot its block table
// gives): the rows come from the lengths' prefix sum, the bounds from the sequence length, the
// query operand tiles are quantized by the workgroup's wavefronts in turn and meet in the LDS,
// the wavefront that scores a page holding a
// new key normalizes, quantizes and inserts that key and scores its own copy of it, and the
// workgroups of chunk 0 write query_starts and row_ends.
//
// MULTI: a request may have more rows than one group (max_query_len > RG), so the pages are
// streamed once per group. Without it the group loop runs once, which the compiler then knows:
// nothing is carried from one group to the next, which took 20-40 registers per wavefront.
//
// SELECT (FUSED one-row groups, one chunk per request): the workgroup holds every key of its
// row, so it also selects the row's top-k from its LDS histogram and its own logits (the
// selection's steps in one workgroup) and writes the positions instead of the workspace
// histograms.
template <int FMT, int H, int RG, int NB, bool HIST, bool FUSED = false, bool MULTI = false,
          bool SELECT = false>
__global__ __launch_bounds__(64 * kWaves) void score_paged_kernel(
    const int32_t *__restrict__ block_table, const int32_t *__restrict__ query_starts,
    int64_t max_blocks, int64_t num_requests, int pages_per_wave,
    const uint8_t *__restrict__ cache, int64_t page_stride, int64_t num_pages, int64_t chunks,
    const uint8_t *__restrict__ q, int64_t q_row_stride, const uint16_t *__restrict__ w,
    int64_t w_row_stride, const int32_t *__restrict__ row_ends, int64_t num_rows,
    int max_query_len, float *__restrict__ logits, int64_t logits_row_stride,
    uint16_t *__restrict__ seghist, uint16_t *__restrict__ coarse, FusedInputs fin,
    int64_t row_lo, int order_work, int select_k, int32_t *__restrict__ select_out,
    int64_t select_stride) {
    static_assert(!FUSED || HIST, "fused inputs: with histograms");
    static_assert(!(FUSED && MULTI), "a fused launch has one row group");
    static_assert(!SELECT || (FUSED && RG == 1), "the selection in the launch: one-row requests");
    constexpr int kStagedKeyBytes = staged_key_bytes<FMT>();
    // HIST: per-row histograms of this workgroup's logits; every wavefront reaches the
    // workgroup barriers below, so no wavefront returns early on a wavefront-level condition
    __shared__ __align__(16) uint32_t hist[HIST ? RG * (kBins / 2) : 1];
    // FUSED: the workgroup's query operands, and each wavefront's staged new keys
    __shared__ __align__(16) uint8_t step_lds_bytes[FUSED ? sizeof(StepQueryLds<FMT, H, RG>) : 16];
    __shared__ __align__(16) uint8_t staged_keys[FUSED ? kWaves * RG * kStagedKeyBytes : 16];
    auto &step_lds = *reinterpret_cast<StepQueryLds<FMT, H, RG> *>(step_lds_bytes);
    // SELECT: the radix select's LDS, the coarse counts, the selection's state, and a copy of
    // the row's logits (every key of the row is this workgroup's: positions below 4096)
    struct SelectState {
        uint32_t bin;
        int above, m;
        uint32_t n_taken;  // keys placed so far: above the bin (low 16 bits), inside it (high)
    };
    __shared__ std::conditional_t<SELECT, SelectShared<64 * kWaves>, int> sel_sh;
    __shared__ uint32_t sel_coarse[SELECT ? kCoarseBins : 1];
    __shared__ SelectState sel_st;
    __shared__ float sel_logits[SELECT ? kWaves * kMaxPagesPerWave * kPageTokens : 1];
    const int lane = threadIdx.x & 63;
    // uniform across the wavefront; said explicitly so that all page and bound arithmetic
    // below stays in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, grp = lane >> 4;
    // byte selectors of tile_scales: rows 0-1 / 2-3, then even / odd rows
    const uint32_t sel32 = lane < 32 ? 0x05040100u : 0x07060302u;
    const uint32_t sel16 = (grp & 1) == 0 ? 0x06020400u : 0x07030501u;
    // Workgroup b takes chunk c = b / R of request (b + c) mod R (R requests; fewer than 2^31
    // workgroups, so 32-bit arithmetic). Workgroups go to the 8 XCDs in turn by index, b mod 8:
    // rotating the requests by one per chunk makes the chunks of one request visit the XCDs in
    // turn, so every XCD gets an equal share of every request's work however the requests'
    // lengths differ, and a grid of one workgroup per compute unit still gives each XCD as many
    // workgroups as it has compute units.
    //
    // Multi-row groups of at most 256 requests and 64 chunks (order_work: not the row tiles of a
    // tiled selection, whose grids are mostly requests outside the tile) instead take the longest-first
    // order (longest_first_item) from the requests' row counts, loaded first: one more round
    // trip before the table slice, against a shorter tail. The fused form also has each
    // request's sequence length, so its chunks past the request's keys are not items at all;
    // the plain form keeps every chunk of a request with rows (those past its keys leave at once).
    const uint32_t R = (uint32_t)num_requests;
    const int PW = pages_per_wave;
    const bool ordered = RG > 1 && order_work != 0 && R <= 256u && chunks <= 64;
    int ord_q[4] = {0, 0, 0, 0}, ord_s[4] = {0, 0, 0, 0};  // FUSED: lengths of request 64 u + lane
    uint32_t chunk32, req32;
    if (ordered) {
        int lvl[4], nch[4];
        const int64_t span = (int64_t)kWaves * PW * kPageTokens;  // keys per chunk
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t qi = 64u * u + (uint32_t)lane;
            const uint32_t qc = qi < R ? qi : R - 1;
            if constexpr (FUSED) {
                ord_q[u] = query_starts[qc];
                ord_s[u] = fin.seq_lens[qc];
            } else {  // query_starts holds the rows' prefix sums
                ord_q[u] = query_starts[qc + 1] - query_starts[qc];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool live = 64u * u + (uint32_t)lane < R;
            int rows_q = live ? ord_q[u] : 0;
            rows_q = rows_q < 0 ? 0 : (rows_q > max_query_len ? max_query_len : rows_q);
            int64_t c = chunks;
            if constexpr (FUSED) {
                const int64_t keys = live && ord_s[u] > 0 ? ord_s[u] : 0;
                c = (keys + span - 1) / span;
            }
            lvl[u] = rows_q > 4 ? 4 : rows_q;
            nch[u] = rows_q > 0 ? (int)(c < chunks ? c : chunks) : 0;
        }
        const WorkItem it = longest_first_item(blockIdx.x, lvl, nch, (uint32_t)chunks);
        chunk32 = __builtin_amdgcn_readfirstlane(it.chunk);
        req32 = __builtin_amdgcn_readfirstlane(it.req);
    } else {
        chunk32 = __builtin_amdgcn_readfirstlane(blockIdx.x / R);
        const uint32_t rot = chunk32 % R;
        req32 = blockIdx.x - chunk32 * R + rot;
        if (req32 >= R) req32 -= R;
    }
    const int64_t chunk = chunk32;
    const int64_t req = req32;
    const int64_t width = max_blocks * kPageTokens;
    // The workgroup's chunk is blocks [chunk_begin, chunk_begin + 4 PW); its wavefronts take
    // them in turn (wavefront w: blocks chunk_begin + w + 4 p), so a chunk that the request's
    // keys only partly fill still gives its four wavefronts equal work.
    const int64_t chunk_begin = chunk * kWaves * (int64_t)PW;
    const int64_t blk_first = chunk_begin + wave;
    auto block_of = [&](int p) -> int64_t { return blk_first + (int64_t)kWaves * p; };
    // At wave launch (every operand is a preloaded argument): this wavefront's slice of the
    // block table (one entry per lane; every entry below max_blocks is in bounds), then the
    // request's rows (nothing before these loads in the kernel writes memory). The table slice
    // goes first because the fused form's first-row sum waits for its own loads, and a wait
    // covers every load issued before it. Then every other argument at once.
    const int32_t *bt = block_table + req * max_blocks;
    const int bt_lane = lane < PW && block_of(lane) < max_blocks ? bt[block_of(lane)] : -1;
    // FUSED one-row groups: the query and head weights of row `req` go out in the same round
    // trip, before the request's first row is known. Where every request has one row (decode)
    // that is its row, and the query's quantization then overlaps the first pages' loads
    // instead of waiting for a second round trip; otherwise they are loaded again below.
    // A launch has at least one row, so `spec_row` is a row of the inputs.
    constexpr bool kSpecQuery = FUSED && RG == 1;
    const int64_t spec_row = req < num_rows ? req : num_rows - 1;
    StepQuery<FMT, H, RG> sq;
    if constexpr (kSpecQuery)
        sq.load(reinterpret_cast<const uint16_t *>(q), q_row_stride, fin.q_head_stride, fin.w_in,
                fin.proj_row_stride, spec_row, spec_row + 1, wave, l16, grp);
    // FUSED: `query_starts` holds the query lengths; the first round of the first-row sum's
    // loads goes out in the same round trip (after the query's, which arrive with them)
    FirstRowLoads first_row_loads;
    if constexpr (FUSED) {
        if (ordered) {
#pragma unroll
            for (int u = 0; u < 4; ++u) first_row_loads.v[u] = ord_q[u];
        } else {
            first_row_loads = issue_first_row(query_starts, num_requests, lane);
        }
    }

    // Table entry of run page p (uniform), or -1 if it names no page of the cache.
    const uint32_t npages = num_pages < INT32_MAX ? (uint32_t)num_pages : (uint32_t)INT32_MAX;
    auto table_page = [&](int p) -> int {
        const int pg = __builtin_amdgcn_readlane(bt_lane, p);
        return (uint32_t)pg < npages ? pg : -1;
    };
    // Section that run page p's loads read: the page itself, or page 0 as a stand-in for a
    // page that is not scored (past `limit`, or not a page of the cache).
    auto section = [&](int p, int limit) {
        const int pg = p < limit ? table_page(p) : -1;
        return cache + (int64_t)(pg >= 0 ? pg : 0) * page_stride;
    };
    const LaneOffsets<FMT> off(l16, grp);
    PageRegs<FMT> buf[NB];

    int64_t r0, r1;
    int qlen = 0, seq = 0;
    if constexpr (!FUSED) {
        r0 = query_starts[req];
        r1 = query_starts[req + 1];
    } else {
        // the request's own length and sequence length are scalar loads
        qlen = query_starts[req];
        seq = fin.seq_lens[req];
        // The first NB - 1 pages go out as soon as the table slice is in, before the first-row
        // sum waits for its loads (issued before them, so that wait does not cover the pages):
        // the pages stream while the rows are found and the query is encoded. A chunk past the
        // request's keys (known below) reads pages it does not score.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int p = 0; p < NB - 1; ++p) load_page(buf[p], section(p, PW), off);
        asm volatile("" ::: "memory");
        r0 = finish_first_row(first_row_loads, query_starts, req, lane);
        r1 = r0 + qlen;
    }
    hoist_args(num_pages, chunks, q, q_row_stride, w, w_row_stride, row_ends, num_rows,
               max_query_len, logits, logits_row_stride, seghist, coarse);
    if constexpr (FUSED) {
        hoist_args(fin.key_in, fin.w_in, fin.proj_row_stride, fin.q_head_stride, fin.gamma,
                   fin.beta, fin.eps, fin.c_h, fin.query_starts, fin.row_ends);
        // decode_layout's outputs (before any early exit): request lq's, from the workgroups
        // of its chunk 0, or in the longest-first order from workgroup lq (every request has a
        // workgroup of that index: the grid holds chunks x R >= R of them)
        int64_t lq = -1, lr0 = 0;
        int lqlen = 0, lseq = 0;
        if (!ordered) {
            if (chunk == 0) {
                lq = req;
                lr0 = r0;
                lqlen = qlen;
                lseq = seq;
            }
        } else if (blockIdx.x < R) {
            lq = blockIdx.x;
            lqlen = request_value(ord_q, (uint32_t)lq);
            lseq = request_value(ord_s, (uint32_t)lq);
            int acc = 0;
#pragma unroll
            for (int u = 0; u < 4; ++u) acc += 64 * u + lane < lq ? ord_q[u] : 0;
            auto add = [](int a, int c) { return a + c; };
            acc = xor_combine<1>(acc, add);
            acc = xor_combine<2>(acc, add);
            acc = xor_combine<4>(acc, add);
            acc = xor_combine<8>(acc, add);
            acc = xor_combine<16>(acc, add);
            acc = xor_combine<32>(acc, add);
            lr0 = __builtin_amdgcn_readfirstlane(acc);
        }
        if (lq >= 0 && wave == 0) {
            if (lq == 0 && lane == 0) fin.query_starts[0] = 0;
            if (lane == 0) fin.query_starts[lq + 1] = (int32_t)(lr0 + lqlen);
            for (int64_t i = lane; lr0 >= 0 && i < lqlen && lr0 + i < num_rows; i += 64) {
                const int64_t e = (int64_t)lseq - lqlen + i + 1;
                fin.row_ends[lr0 + i] = (int32_t)(e < 0 ? 0 : e);
            }
            if (lq == (int64_t)R - 1) {  // rows from query_starts[R] on are graph padding
                const int64_t total = lr0 + lqlen;
                for (int64_t row = (total > 0 ? total : 0) + lane; row < num_rows; row += 64)
                    fin.row_ends[row] = 0;
            }
        }
        if constexpr (SELECT) {  // ... which select nothing (the whole workgroup writes them)
            if (lq == (int64_t)R - 1) {
                const int64_t total = lr0 + lqlen;
                for (int64_t row = total > 0 ? total : 0; row < num_rows; ++row)
                    for (int i = threadIdx.x; i < select_k; i += 64 * kWaves)
                        select_out[row * select_stride + i] = -1;
            }
        }
    }

    if (r0 < 0) return;
    if (r1 > r0 + max_query_len) r1 = r0 + max_query_len;
    // the row window [row_lo, num_rows): rows outside it are neither scored nor written, and
    // the logits and histograms of row r go to row r - row_lo of their buffers (row_lo is 0
    // except for the tiles of a row-tiled selection)
    if (r1 > num_rows) r1 = num_rows;
    if (r0 < row_lo) r0 = row_lo;
    const int nrows = (int)(r1 - r0);
    if (nrows <= 0) return;

    // Query operands of the first row group, in flight together with the row bounds.
    const int ngroups = MULTI ? (nrows + RG - 1) / RG : 1;  // nrows <= max_query_len <= RG otherwise
    // the fused operands of four-row MXFP4 groups and two-row FP8 groups (FP8 operands are
    // widened to BF16, twice the registers) stay in the LDS
    RowGroup<FMT, H, RG, FUSED && (RG == 4 || (is_fp8(FMT) && RG == 2))> rows;
    int kmax;
    // FUSED: the step's keys (one row each; a key past the rows reads the first row's)
    KeyLane key;  // columns 2 lane, 2 lane + 1 of the LayerNorm weights and biases
    uint32_t key_pair[FUSED ? RG : 1];
    if constexpr (!FUSED) {
        rows.load(q, q_row_stride, w, w_row_stride, row_ends, r0, r1, width, l16, grp);
        // Keys this request needs: the largest bound over its rows.
        kmax = lane < nrows ? row_ends[r0 + lane] : 0;
    } else {
        const int64_t e = (int64_t)seq - qlen + nrows;  // the last row's bound is the largest
        kmax = (int)(e < 0 ? 0 : (e > width ? width : e));
        // the bounds need no loads here: a chunk past the request's keys leaves before any
        // query work (no new key lies in it: every key's position is below the last bound);
        // SELECT: its one chunk has no keys, the row selects none
        if (chunk_begin * kPageTokens >= kmax) {
            if constexpr (SELECT)
                for (int i = threadIdx.x; i < select_k; i += 64 * kWaves)
                    select_out[r0 * select_stride + i] = -1;
            return;
        }
        if (!kSpecQuery || r0 != spec_row)
            sq.load(reinterpret_cast<const uint16_t *>(q), q_row_stride, fin.q_head_stride,
                    fin.w_in, fin.proj_row_stride, r0, r1, wave, l16, grp);
        key = load_key(fin.key_in + r0 * fin.proj_row_stride, fin.gamma, fin.beta, nullptr, lane);
        key_pair[0] = key.pair;
#pragma unroll
        for (int i = 1; i < RG; ++i)
            key_pair[i] = *reinterpret_cast<const uint32_t *>(
                fin.key_in + (r0 + (i < nrows ? i : 0)) * fin.proj_row_stride + 2 * lane);
    }

    // The plain form's first NB - 1 pages go out after the query and bound loads: loads
    // complete in issue order, so the first page's math then waits for that page and not for
    // the whole ring.
    if constexpr (!FUSED) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int p = 0; p < NB - 1; ++p) load_page(buf[p], section(p, PW), off);
        asm volatile("" ::: "memory");
    }

    // FUSED: the new key at position seq - qlen + i belongs to the wavefront whose run holds
    // its block. The step's keys are consecutive positions (at most 4), so they span at most
    // two consecutive blocks, which belong to different wavefronts: a wavefront owns at most
    // one page of new keys (own_pp, its run page, or -1; own_mask, the keys on it). It
    // normalizes, quantizes and inserts those keys, keeps a copy in the LDS, and loads the page
    // once more for itself: that copy takes the new keys and is scored on its own, and the
    // ring skips the page, so that the ring's registers are never rewritten (rewriting them
    // in place made the compiler wait for each page's loads as soon as they were issued).
    int own_pp = -1;
    uint32_t own_mask = 0;
    int own_o[FUSED ? RG : 1];
    PageRegs<FMT> own_pg;
    if constexpr (FUSED) {
#pragma unroll
        for (int i = 0; i < RG; ++i) {
            own_o[i] = 0;
            const int64_t pos = (int64_t)seq - qlen + i;
            if (i >= nrows || pos < 0 || pos >= width) continue;
            const int64_t rel = (pos >> 6) - chunk_begin;
            if (rel < 0 || rel >= kWaves * (int64_t)PW || (rel & (kWaves - 1)) != wave) continue;
            if (table_page((int)(rel / kWaves)) < 0) continue;
            own_pp = (int)(rel / kWaves);
            own_mask |= 1u << i;
            own_o[i] = (int)(pos & 63);
        }
        // issued by every wavefront (a non-owner reads its first ring page again, which the
        // ring is loading anyway), so that no branch joins around loads in flight
        load_page(own_pg, section(own_pp >= 0 ? own_pp : 0, PW), off);
        sq.encode(step_lds, fin.c_h, wave, lane);
        if (own_pp >= 0) {
            uint8_t *sec = const_cast<uint8_t *>(section(own_pp, PW));  // the caller's writable cache
#pragma unroll
            for (int i = 0; i < RG; ++i) {
                if (!((own_mask >> i) & 1u)) continue;
                KeyLane k = key;
                k.pair = key_pair[i];
                float n0, n1;
                layer_norm_pair(k, fin.eps, n0, n1);
                uint8_t *staged = staged_keys + (wave * RG + i) * kStagedKeyBytes;
                if constexpr (FMT == kFmtMxfp4) {
                    const Mxfp4KeyLane mk = mxfp4_key_lane(n0, n1);
                    store_mxfp4_key(mk, sec, own_o[i], lane);
                    staged[lane] = (uint8_t)mk.byte;
                    if ((lane & 15) == 0) staged[64 + (lane >> 4)] = (uint8_t)mk.scale;
                } else {
                    const Fp8KeyLane fk = fp8_key_lane(n0, n1);
                    store_fp8_key<FMT>(fk, sec, own_o[i], lane);
                    *reinterpret_cast<uint16_t *>(staged + 2 * lane) = (uint16_t)fk.two;
                    if (lane == 0) *reinterpret_cast<uint32_t *>(staged + 128) = fp8_scale_word<FMT>(fk.s);
                }
            }
        }
        __syncthreads();
        rows.from_lds(step_lds, r0, seq, qlen, r0, r1, width, lane);
    }
    kmax = group_max<64>(kmax);
    kmax = __builtin_amdgcn_readfirstlane(kmax);
    const int64_t kext = kmax < width ? kmax : width;
    const int64_t nblk = (kext + kPageTokens - 1) / kPageTokens;
    // a chunk past the request's keys has nothing to score and no histogram to write (the
    // selection reads only segments that hold keys of the row): the whole workgroup leaves
    if (chunk_begin >= nblk) {
        if constexpr (SELECT)  // (not reached: kmax > 0 above)
            for (int i = threadIdx.x; i < select_k; i += 64 * kWaves)
                select_out[r0 * select_stride + i] = -1;
        return;
    }
    const int64_t chunk_end = chunk_begin + kWaves * (int64_t)PW < nblk
                                  ? chunk_begin + kWaves * (int64_t)PW : nblk;
    // pages of this wavefront below chunk_end
    const int run = blk_first < chunk_end ? (int)((chunk_end - blk_first + kWaves - 1) / kWaves) : 0;

    // SELECT: the top-k of the row (bound n) into out[0..k), from the workgroup's LDS histogram
    // and LDS copy of the row's logits (every key of the row is this workgroup's) -- the
    // selection's steps in one workgroup: the coarse bin holding the k-th largest key, the fine
    // bin inside it, then each wavefront's keys above the bin to the output and inside it to a
    // candidate list in the histogram's LDS, and the candidates' radix select (one wavefront's
    // for at most 64).
    auto select_row = [&](int64_t n, int64_t row) {
        if constexpr (SELECT) {
            int32_t *out = select_out + row * select_stride;
            const int k = select_k;
            if (n <= k) {
                for (int i = threadIdx.x; i < k; i += 64 * kWaves) out[i] = i < n ? (int32_t)i : -1;
                return;
            }
            {  // coarse bin c = the 64 fine bins of lanes 4 c .. 4 c + 3
                const uint4 *src = reinterpret_cast<const uint4 *>(hist) + 2 * threadIdx.x;
                const uint4 a = src[0], b = src[1];
                const uint32_t w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                uint32_t s16 = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) s16 += (w8[e] & 0xFFFFu) + (w8[e] >> 16);
                s16 += lane_xor<1>(s16);
                s16 += lane_xor<2>(s16);
                if ((threadIdx.x & 3) == 0) sel_coarse[threadIdx.x >> 2] = s16;
            }
            __syncthreads();
            if (wave == 0) {  // lane l: coarse bin 63 - l, then fine bin 63 - l of the coarse bin
                const Found64 fc = find_in_64_wave(sel_coarse[63 - lane], k);
                const uint32_t B = 63u - (uint32_t)fc.lane;
                const uint32_t fb = B * 64u + (63u - (uint32_t)lane);
                const uint32_t cnt = (hist[fb >> 1] >> (16u * (fb & 1u))) & 0xFFFFu;
                const Found64 ff = find_in_64_wave(cnt, k - fc.before);
                if (lane == 0) {
                    sel_st.bin = B * 64u + 63u - (uint32_t)ff.lane;
                    sel_st.above = fc.before + ff.before;
                    sel_st.m = (int)ff.count;
                    sel_st.n_taken = 0;
                }
            }
            __syncthreads();
            const uint32_t bin = sel_st.bin;
            const int above = sel_st.above, m = sel_st.m, r = k - above;  // 1 <= r <= m
            int pos_bits = 1;
            while (pos_bits < 31 && ((int64_t)1 << pos_bits) < n) ++pos_bits;
            uint64_t *cands = reinterpret_cast<uint64_t *>(hist);  // the histogram is read
            constexpr int kCap = (int)(sizeof(hist) / (sizeof(uint64_t)));
            for (int p = 0; p < run; ++p) {  // (no register array indexed by p: not unrolled)
                if (table_page(p) < 0) continue;  // uniform
                const int64_t kb = block_of(p) * kPageTokens;
                const bool live = (int64_t)lane < n - kb;
                const uint32_t u = order_key(sel_logits[kb + lane]);
                const bool ab = live && (u >> kBinShift) > bin;
                const bool in = live && (u >> kBinShift) == bin;
                const uint32_t pos = (uint32_t)kb + (uint32_t)lane;
                // both slots from one atomic on the packed counts (each below 2^16: n <= 4096)
                const uint64_t mab = __ballot(ab), min_ = __ballot(in);
                uint32_t base = 0;
                if (mab | min_) {
                    if (lane == 0)
                        base = atomicAdd(&sel_st.n_taken,
                                         (uint32_t)__builtin_popcountll(mab) |
                                             ((uint32_t)__builtin_popcountll(min_) << 16));
                    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
                }
                const uint32_t sa = (base & 0xFFFFu) + lanes_below(mab);
                const uint32_t sc = (base >> 16) + lanes_below(min_);
                if (ab && sa < (uint32_t)above) out[sa] = (int32_t)pos;
                if (in) {
                    if (r == m) {  // every key inside the bin is taken
                        if (above + (int)sc < k) out[above + sc] = (int32_t)pos;
                    } else if (sc < (uint32_t)kCap) {
                        cands[sc] = composite(u, pos, pos_bits);
                    }
                }
            }
            if (r == m) return;
            __syncthreads();  // the candidates are in the LDS
            const int bits = 20 + pos_bits;
            if (m <= 64) {
                if (wave == 0) wave_select_out(cands, m, r, bits, pos_bits, out + above);
            } else if (m <= kCap) {
                select_smallest(LdsCandidates<64 * kWaves>{cands, m}, r, bits, pos_bits, out + above,
                                sel_sh);
            } else {  // the bin overflowed the list: its keys again from the logits' copy
                select_smallest(RowBin<64 * kWaves>{sel_logits, n, bin, pos_bits}, r, bits,
                                pos_bits, out + above, sel_sh);
            }
        }
    };

    // Requests with more rows than one register group stream their pages once per group
    // (the second and later passes mostly hit the L2).
    for (int g = 0; g < ngroups; ++g) {
        const int64_t first = r0 + (int64_t)g * RG;
        if (g > 0) {
            if constexpr (!FUSED)  // a fused launch has a single row group
                rows.load(q, q_row_stride, w, w_row_stride, row_ends, first, r1, width, l16, grp);
#pragma unroll
            for (int p = 0; p < NB - 1; ++p) load_page(buf[p], section(p, run), off);
        }
        const int count = (int)(r1 - first);
        if constexpr (HIST) {
            __syncthreads();  // the previous group's histograms are written out
            for (int i = threadIdx.x; i < RG * (kBins / 2); i += 64 * kWaves) hist[i] = 0;
            __syncthreads();
        }
        if constexpr (FUSED) {  // the page of new keys (a fused launch has one row group)
            if (own_pp >= 0) {
#pragma unroll
                for (int i = 0; i < RG; ++i)
                    if ((own_mask >> i) & 1u)
                        patch_key(own_pg, staged_keys + (wave * RG + i) * kStagedKeyBytes,
                                  own_o[i], l16, grp);
                rows.score(own_pg, (int)(block_of(own_pp) * kPageTokens), count, logits,
                           first - row_lo, logits_row_stride, lane, grp, HIST ? hist : nullptr,
                           sel32, sel16, SELECT ? sel_logits : nullptr);
            }
        }
        for (int base = 0; base < run; base += NB) {
#pragma unroll
            for (int slot = 0; slot < NB; ++slot) {
                // keep the ring as written: without this compiler-only fence (it emits
                // nothing) later pages' loads get hoisted, which costs the registers a second
                // wavefront per SIMD needs to overlap one wavefront's math with another's loads
                asm volatile("" ::: "memory");
                const int p = base + slot;
                load_page(buf[(slot + NB - 1) % NB], section(p + NB - 1, run), off);
                if (p < run && table_page(p) >= 0 && (!FUSED || p != own_pp))
                    rows.score(buf[slot], (int)(block_of(p) * kPageTokens), count, logits,
                               first - row_lo, logits_row_stride, lane, grp,
                               HIST ? hist : nullptr, sel32, sel16,
                               SELECT ? sel_logits : nullptr);
            }
        }
        if constexpr (SELECT) {
            __syncthreads();  // the row's histogram is complete
            select_row(rows.rend[0], first);
        } else if constexpr (HIST) {
            // (row, segment = chunk) histograms of the rows whose keys reach this chunk; the
            // packed 16-bit counts are already the workspace's layout
            __syncthreads();
            const int64_t seg_begin = chunk_begin * kPageTokens;
#pragma unroll
            for (int j = 0; j < RG; ++j) {  // unrolled: a runtime index would put `rows` in scratch
                if (j >= count || seg_begin >= rows.rend[j]) continue;
                // lane t copies fine bins [16 t, 16 t + 16) and, with lanes 4c..4c+3, forms
                // coarse bin c (fine bins [64 c, 64 c + 64))
                const int64_t at = (first + j - row_lo) * chunks + chunk;
                uint4 *dst = reinterpret_cast<uint4 *>(seghist + at * kBins) + 2 * threadIdx.x;
                const uint4 *src = reinterpret_cast<const uint4 *>(hist + j * (kBins / 2)) +
                                   2 * threadIdx.x;
                const uint4 a = src[0], b = src[1];
                uint32_t s16 = 0;
                const uint32_t w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) s16 += (w8[e] & 0xFFFFu) + (w8[e] >> 16);
                s16 += lane_xor<1>(s16);
                s16 += lane_xor<2>(s16);
                // a fine block goes out only where its coarse count is nonzero (most of the
                // 64 are empty); the selection reads a block only where the count says so
                if (s16 != 0) {
                    dst[0] = a;
                    dst[1] = b;
                }
                if ((threadIdx.x & 3) == 0)
                    coarse[at * kCoarseBins + (threadIdx.x >> 2)] = (uint16_t)s16;
            }
        }
    }
}

int device_cus() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Pages per wavefront: about one wavefront per SIMD (four per compute unit) over the whole
// (request x block) space, 1 to 16 pages (a multiple of 4 above 4). Fewer, longer wavefronts
// measured faster than two or more per SIMD: each wavefront's start (row bounds, query
// operands, first pages) and histogram flush is paid fewer times, and one wavefront's loads in
// flight already cover the memory latency. A small workload spreads over more wavefronts with
// fewer pages each: the launch is then as long as one wavefront's start and few pages.
int score_pages_per_wave(int64_t num_requests, int64_t max_blocks) {
    const int64_t target_waves = (int64_t)device_cus() * kWaves;
    int64_t ppw = (num_requests * max_blocks + target_waves - 1) / target_waves;
    if (ppw > 4) ppw = (ppw + 3) / 4 * 4;
    int p = (int)(ppw < 1 ? 1 : (ppw > kMaxPagesPerWave ? kMaxPagesPerWave : ppw));
    // a row spans at most kMaxRowSegments scoring workgroups
    while (p < kMaxPagesPerWave && (max_blocks + kWaves * p - 1) / (kWaves * p) > kMaxRowSegments)
        p = p < 4 ? p + 1 : p + 4;
    return p;
}

ScoreGeometry score_geometry(int64_t num_requests, int64_t max_blocks) {
    ScoreGeometry g;
    g.pages_per_wave = score_pages_per_wave(num_requests, max_blocks);
    const int64_t pages_per_wg = (int64_t)kWaves * g.pages_per_wave;
    g.chunks = (max_blocks + pages_per_wg - 1) / pages_per_wg;
    g.segment_keys = pages_per_wg * kPageTokens;
    return g;
}

template <int FMT, int H, int RG, bool HIST, bool FUSED = false, bool MULTI = false,
          bool SELECT = false>
static hipError_t launch_score_rg(const ScoreArgs &a, const TopkWorkspace &ws, hipStream_t stream,
                                  const FusedInputs &fin = FusedInputs{}) {
    const ScoreGeometry geo = score_geometry(a.geometry_requests > 0 ? a.geometry_requests
                                                                     : a.num_requests,
                                             a.max_blocks);
    const dim3 grid((unsigned)(geo.chunks * a.num_requests)), block(64 * kWaves);
    // page buffers per wavefront: 3 for MXFP4 (measured best of 2-6 on the long-context
    // workload, and better than 2 on the verify workload's 4-row groups), else 2 (FP8 pages
    // take the registers a deeper ring would need)
    constexpr int NB = FMT == kFmtMxfp4 ? 3 : 2;
    hipLaunchKernelGGL((score_paged_kernel<FMT, H, RG, NB, HIST, FUSED, MULTI, SELECT>), grid, block, 0, stream,
                       a.block_table, a.query_starts, a.max_blocks, a.num_requests,
                       geo.pages_per_wave, static_cast<const uint8_t *>(a.cache), a.page_stride,
                       a.num_pages, geo.chunks, static_cast<const uint8_t *>(a.q), a.q_row_stride,
                       static_cast<const uint16_t *>(a.w), a.w_row_stride, a.row_ends,
                       a.num_rows, a.max_query_len, a.logits, a.logits_row_stride, ws.seghist,
                       ws.coarse, fin, a.row_lo, a.geometry_requests > 0 ? 0 : 1, a.select_k,
                       a.select_out, a.select_stride);
    return hipGetLastError();
}

template <int FMT, int H, bool HIST>
static hipError_t launch_score_h(const ScoreArgs &a, const TopkWorkspace &ws, hipStream_t stream) {
    if (a.max_query_len <= 1) return launch_score_rg<FMT, H, 1, HIST>(a, ws, stream);
    if constexpr (is_fp8(FMT)) {
        // FP8 queries occupy 4x the registers once widened to BF16: at most 2 rows per group
        if (a.max_query_len <= 2) return launch_score_rg<FMT, H, 2, HIST>(a, ws, stream);
        return launch_score_rg<FMT, H, 2, HIST, false, true>(a, ws, stream);
    } else {
        if (a.max_query_len <= 2) return launch_score_rg<FMT, H, 2, HIST>(a, ws, stream);
        if (a.max_query_len <= 4) return launch_score_rg<FMT, H, 4, HIST>(a, ws, stream);
        return launch_score_rg<FMT, H, 4, HIST, false, true>(a, ws, stream);
    }
}

template <int FMT, bool HIST>
static hipError_t launch_score_fmt(const ScoreArgs &a, const TopkWorkspace &ws, hipStream_t stream) {
    switch (a.heads) {
        case 16: return launch_score_h<FMT, 16, HIST>(a, ws, stream);
        case 32: return launch_score_h<FMT, 32, HIST>(a, ws, stream);
        default: return launch_score_h<FMT, 64, HIST>(a, ws, stream);
    }
}

hipError_t launch_score_paged(const ScoreArgs &a, hipStream_t stream) {
    switch (a.fmt) {
        case kFmtMxfp4: return launch_score_fmt<kFmtMxfp4, false>(a, TopkWorkspace{}, stream);
        case kFmtFp8: return launch_score_fmt<kFmtFp8, false>(a, TopkWorkspace{}, stream);
        default: return launch_score_fmt<kFmtFp8Mx, false>(a, TopkWorkspace{}, stream);
    }
}

size_t score_topk_workspace_bytes(int64_t num_requests, int64_t max_blocks, int64_t num_rows) {
    return topk_layout_bytes(num_rows, score_geometry(num_requests, max_blocks).chunks);
}

hipError_t launch_score_paged_hist(const ScoreArgs &a, void *workspace, hipStream_t stream) {
    const ScoreGeometry geo = score_geometry(a.num_requests, a.max_blocks);
    const TopkWorkspace ws = carve(workspace, a.num_rows, geo.chunks);
    switch (a.fmt) {
        case kFmtMxfp4: return launch_score_fmt<kFmtMxfp4, true>(a, ws, stream);
        case kFmtFp8: return launch_score_fmt<kFmtFp8, true>(a, ws, stream);
        default: return launch_score_fmt<kFmtFp8Mx, true>(a, ws, stream);
    }
}

// Row-tiled scoring and selection: for each tile of `tile_rows` consecutive rows, the scorer
// with that row window (logits and histograms in tile-row order, so both buffers hold one
// tile), then the rest of the selection on the tile's rows. A tile holds the rows of about
// tile_rows / max_query_len requests (at least that many when requests have their most rows),
// so the scorer's geometry is sized for that many: a tile's pages spread over about one
// wavefront per SIMD, as a whole batch's do.
int64_t tiled_geometry_requests(int64_t num_requests, int64_t tile_rows, int max_query_len) {
    const int64_t per = (tile_rows + max_query_len - 1) / max_query_len;
    return per < num_requests ? per : num_requests;
}

size_t score_topk_tiled_workspace_bytes(int64_t num_requests, int64_t max_blocks,
                                        int64_t tile_rows, int max_query_len) {
    const int64_t gr = tiled_geometry_requests(num_requests, tile_rows, max_query_len);
    return topk_layout_bytes(tile_rows, score_geometry(gr, max_blocks).chunks);
}

hipError_t launch_score_topk_tiled(const ScoreArgs &base, int k, int32_t *indices,
                                   int64_t indices_row_stride, int64_t tile_rows,
                                   void *workspace, hipStream_t stream) {
    const int64_t gr = tiled_geometry_requests(base.num_requests, tile_rows, base.max_query_len);
    const ScoreGeometry geo = score_geometry(gr, base.max_blocks);
    const int64_t width = base.max_blocks * kPageTokens;
    for (int64_t lo = 0; lo < base.num_rows; lo += tile_rows) {
        const int64_t hi = lo + tile_rows < base.num_rows ? lo + tile_rows : base.num_rows;
        // laid out for the tile's own row count, as the selection below carves it (the last
        // tile may be shorter; a shorter layout fits in the space of a full one)
        const TopkWorkspace ws = carve(workspace, hi - lo, geo.chunks);
        ScoreArgs a = base;
        a.geometry_requests = gr;
        a.row_lo = lo;
        a.num_rows = hi;
        hipError_t e;
        switch (a.fmt) {
            case kFmtMxfp4: e = launch_score_fmt<kFmtMxfp4, true>(a, ws, stream); break;
            case kFmtFp8: e = launch_score_fmt<kFmtFp8, true>(a, ws, stream); break;
            default: e = launch_score_fmt<kFmtFp8Mx, true>(a, ws, stream); break;
        }
        if (e != hipSuccess) return e;
        e = launch_topk_after_histograms(base.logits, hi - lo, width, base.logits_row_stride,
                                         base.row_ends + lo, k, indices + lo * indices_row_stride,
                                         indices_row_stride, workspace, geo.chunks,
                                         geo.segment_keys, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// The step's inputs and its scoring in one launch (histograms, one row group: at most 4 rows
// per request for MXFP4, 2 for FP8, whose widened operands take twice the registers).
template <int FMT, int H>
static hipError_t launch_index_score_h(const ScoreArgs &a, const FusedInputs &fin,
                                       const TopkWorkspace &ws, hipStream_t stream) {
    if (a.max_query_len <= 1) return launch_score_rg<FMT, H, 1, true, true>(a, ws, stream, fin);
    if constexpr (FMT == kFmtMxfp4) {
        if (a.max_query_len <= 2) return launch_score_rg<FMT, H, 2, true, true>(a, ws, stream, fin);
        return launch_score_rg<FMT, H, 4, true, true>(a, ws, stream, fin);
    } else {
        return launch_score_rg<FMT, H, 2, true, true>(a, ws, stream, fin);
    }
}

template <int FMT>
static hipError_t launch_index_score_fmt(const ScoreArgs &a, const FusedInputs &fin,
                                         const TopkWorkspace &ws, hipStream_t stream) {
    switch (a.heads) {
        case 16: return launch_index_score_h<FMT, 16>(a, fin, ws, stream);
        case 32: return launch_index_score_h<FMT, 32>(a, fin, ws, stream);
        default: return launch_index_score_h<FMT, 64>(a, fin, ws, stream);
    }
}

int index_score_max_query_len(int fmt) { return fmt == kFmtMxfp4 ? 4 : 2; }

hipError_t launch_index_score_hist(const ScoreArgs &a, const FusedInputs &fin, void *workspace,
                                   hipStream_t stream) {
    if (a.max_query_len < 1 || a.max_query_len > index_score_max_query_len(a.fmt))
        return hipErrorInvalidValue;
    const ScoreGeometry geo = score_geometry(a.num_requests, a.max_blocks);
    const TopkWorkspace ws = carve(workspace, a.num_rows, geo.chunks);
    switch (a.fmt) {
        case kFmtMxfp4: return launch_index_score_fmt<kFmtMxfp4>(a, fin, ws, stream);
        case kFmtFp8: return launch_index_score_fmt<kFmtFp8>(a, fin, ws, stream);
        default: return launch_index_score_fmt<kFmtFp8Mx>(a, fin, ws, stream);
    }
}

// The step with its selection made in the scoring launch (one-row requests, one chunk each):
// score_paged_kernel<..., SELECT = true>.
template <int FMT>
static hipError_t launch_index_select_fmt(const ScoreArgs &a, const FusedInputs &fin,
                                          hipStream_t stream) {
    switch (a.heads) {
        case 16: return launch_score_rg<FMT, 16, 1, true, true, false, true>(a, TopkWorkspace{}, stream, fin);
        case 32: return launch_score_rg<FMT, 32, 1, true, true, false, true>(a, TopkWorkspace{}, stream, fin);
        default: return launch_score_rg<FMT, 64, 1, true, true, false, true>(a, TopkWorkspace{}, stream, fin);
    }
}

hipError_t launch_index_score_topk(const ScoreArgs &a, const FusedInputs &fin, void *workspace,
                                   hipStream_t stream) {
    const ScoreGeometry geo = score_geometry(a.num_requests, a.max_blocks);
    if (a.max_query_len <= 1 && geo.chunks == 1) {
        switch (a.fmt) {
            case kFmtMxfp4: return launch_index_select_fmt<kFmtMxfp4>(a, fin, stream);
            case kFmtFp8: return launch_index_select_fmt<kFmtFp8>(a, fin, stream);
            default: return launch_index_select_fmt<kFmtFp8Mx>(a, fin, stream);
        }
    }
    hipError_t e = launch_index_score_hist(a, fin, workspace, stream);
    if (e != hipSuccess) return e;
    return launch_topk_after_histograms(a.logits, a.num_rows, a.max_blocks * kPageTokens,
                                        a.logits_row_stride, fin.row_ends, a.select_k,
                                        a.select_out, a.select_stride, workspace, geo.chunks,
                                        geo.segment_keys, stream);
}

}  // namespace dsaidx
