// Query quantization and key LayerNorm + quantization + paged insert for gfx950.
//
// quantize_queries: page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index",
//   quantize_fp4_query (MXFP4 of one head; scales after all payload bytes) and
//   DsaIndex.fp8_query (FP8 with one power-of-two scale per head folded into the weight);
//   page "vllm.models.kimi_k3.amd.ops.fp4_indexer", quantize_queries (shape rules).
// index_inputs: same index page, DsaIndex (both of the above for one token per workgroup,
//   reading the head weights and the key from the packed projection row).
// store_keys: same index page, insert_key (FP32 LayerNorm, BF16, then the cache writer; with
//   mx the FP8 scale's exponent as four equal UE8M0 bytes) and insert_fp4_key (payload at
//   token * 64, four UE8M0 bytes at 64 * 64 + token * 4);
//   fp4_indexer page, store_keys (negative slots are padding) and cache_views (sections
//   inside merged pages, addressed by the physical page stride).
//
// Every float operation that decides a stored byte is a single IEEE RN operation written
// with the __f*_rn intrinsics, so the bytes do not depend on contraction choices.
#include "device_common.h"
#include "launch.h"
#include "key_norm.h"
#include "layout.h"

namespace dsaidx {

// One query row of H heads (16, 32 or 64) on a workgroup of 256 lanes (4 wavefronts). Lane t
// owns 8 consecutive columns (one 16-byte load) of head (t / 16) + 16 * pass: 16 lanes per
// head, 4 lanes per 32-value MX block, every lane busy in each of the H / 16 passes.
// The row's loads are one step and its quantization another, so a kernel can issue other
// loads in between.
template <int H>
struct QueryLoads {
    static constexpr int kPasses = H / 16;
    uint4 raws[kPasses];
    uint32_t wraw[kPasses];  // 32-bit: 16-bit lanes would be packed in pairs, which waits for the loads

    // Every pass's 16-byte load is issued before any is used, with no branch around them: the
    // row costs one memory round trip (the head weights, raw with unit head stride, likewise).
    __device__ __forceinline__ void load(const uint16_t *__restrict__ q_row, int64_t q_head_stride,
                                         int tid) {
        const int part = tid & 15;
#pragma unroll
        for (int pass = 0; pass < kPasses; ++pass) {
            const int head = (tid >> 4) + 16 * pass;
            raws[pass] = *reinterpret_cast<const uint4 *>(q_row + (int64_t)head * q_head_stride + part * 8);
        }
    }
    __device__ __forceinline__ void load_weights(const uint16_t *__restrict__ wv_row, int tid) {
#pragma unroll
        for (int pass = 0; pass < kPasses; ++pass)
            wraw[pass] = (uint32_t)wv_row[(tid >> 4) + 16 * pass];
    }
};

template <int FMT, int H>
__device__ __forceinline__ void quantize_query_row(const QueryLoads<H> &in, bool has_w,
                                                   uint8_t *__restrict__ out_row,
                                                   uint16_t *__restrict__ w_out_row, float c_h,
                                                   int tid) {
    constexpr int heads = H, kPasses = H / 16;
    const int part = tid & 15;
    const uint32_t *wraw = in.wraw;
    const uint4 *raws = in.raws;
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
        const int head = (tid >> 4) + 16 * pass;
        const uint4 raw = raws[pass];
        float v[8] = {bf16_lo(raw.x), bf16_hi(raw.x), bf16_lo(raw.y), bf16_hi(raw.y),
                      bf16_lo(raw.z), bf16_hi(raw.z), bf16_lo(raw.w), bf16_hi(raw.w)};
        if constexpr (FMT == kFmtMxfp4) {
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
            amax = group_max<4>(amax);  // the 4 lanes of one 32-value block
            const int e = ue8m0_exponent(amax);
            uint32_t word = 0;  // E2M1 of v * 2^-e, straight from the BF16 pairs
            word = e2m1_bf16_pair<0>(word, raw.x, e);
            word = e2m1_bf16_pair<1>(word, raw.y, e);
            word = e2m1_bf16_pair<2>(word, raw.z, e);
            word = e2m1_bf16_pair<3>(word, raw.w, e);
            *reinterpret_cast<uint32_t *>(out_row + head * 64 + part * 4) = word;
            // UE8M0 bytes of blocks 0..3 live in lanes part = 0, 4, 8, 12 of the head.
            const uint32_t byte = (uint32_t)(e + 127);
            const uint32_t b1 = row_down<4>(byte), b2 = row_down<8>(byte),
                           b3 = row_down<12>(byte);
            if (part == 0) {
                *reinterpret_cast<uint32_t *>(out_row + heads * 64 + head * 4) =
                    byte | (b1 << 8) | (b2 << 16) | (b3 << 24);
                if (has_w) {
                    const float w = bf16_val((uint16_t)wraw[pass]);
                    w_out_row[head] = (uint16_t)bf16_bits_rne(__fmul_rn(w, c_h));
                }
            }
        } else {
            float amax = 1e-10f;
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
            amax = group_max<16>(amax);  // the 16 lanes of the head
            const float s = pow2_ceil(__fdiv_rn(amax, 448.0f));
            const float inv = __fdiv_rn(1.0f, s);
            const uint32_t lo = e4m3x4(__fmul_rn(v[0], inv), __fmul_rn(v[1], inv),
                                       __fmul_rn(v[2], inv), __fmul_rn(v[3], inv));
            const uint32_t hi = e4m3x4(__fmul_rn(v[4], inv), __fmul_rn(v[5], inv),
                                       __fmul_rn(v[6], inv), __fmul_rn(v[7], inv));
            *reinterpret_cast<uint2 *>(out_row + head * 128 + part * 8) = make_uint2(lo, hi);
            if (part == 0 && has_w) {
                const float w = bf16_val((uint16_t)wraw[pass]);
                w_out_row[head] = (uint16_t)bf16_bits_rne(__fmul_rn(__fmul_rn(w, s), c_h));
            }
        }
    }
}

// One key on one wavefront (the LayerNorm and MXFP4 steps live in key_norm.h, shared with the
// scorer that inserts a step's keys itself). Slots outside [0, num_pages * 64) (negative slots
// are padding) write nothing.
template <int FMT>
__device__ __forceinline__ void store_key(const KeyLane &in, float eps,
                                          uint8_t *__restrict__ cache, int64_t num_pages,
                                          int64_t page_stride, int lane) {
    const int64_t slot = in.slot;
    if (slot < 0 || slot >= num_pages * kPageTokens) return;
    float n0, n1;
    layer_norm_pair(in, eps, n0, n1);

    uint8_t *sec = cache + (slot >> 6) * page_stride;
    const int off = (int)(slot & 63);
    if constexpr (FMT == kFmtMxfp4) {
        store_mxfp4_key(mxfp4_key_lane(n0, n1), sec, off, lane);
    } else {
        store_fp8_key<FMT>(fp8_key_lane(n0, n1), sec, off, lane);
    }
}

// The kernels list first the arguments their first loads need: the library is built to
// preload the leading kernel arguments into scalar registers at wave launch.

// One workgroup per query row.
template <int FMT, int H>
__global__ __launch_bounds__(256) void quantize_queries_kernel(
    const uint16_t *__restrict__ q, int64_t q_row_stride, int64_t q_head_stride,
    const uint16_t *__restrict__ wv, int64_t wv_row_stride, uint8_t *__restrict__ q_out,
    int64_t q_out_row_stride, uint16_t *__restrict__ w_out, int64_t w_out_row_stride, float c_h) {
    const int64_t row = blockIdx.x;
    QueryLoads<H> in;
    in.load(q + row * q_row_stride, q_head_stride, threadIdx.x);
    if (wv) in.load_weights(wv + row * wv_row_stride, threadIdx.x);
    quantize_query_row<FMT, H>(in, wv != nullptr, q_out + row * q_out_row_stride,
                               w_out ? w_out + row * w_out_row_stride : nullptr, c_h, threadIdx.x);
}

// One wavefront per key, four keys per workgroup.
template <int FMT>
__global__ __launch_bounds__(256) void store_keys_kernel(
    const uint16_t *__restrict__ keys, int64_t k_row_stride, int64_t tokens,
    const float *__restrict__ gamma, const float *__restrict__ beta,
    const int64_t *__restrict__ slots, uint8_t *__restrict__ cache, float eps, int64_t num_pages,
    int64_t page_stride) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= tokens) return;
    const int lane = threadIdx.x & 63;
    store_key<FMT>(load_key(keys + t * k_row_stride, gamma, beta, slots + t, lane), eps, cache,
                   num_pages, page_stride, lane);
}

// Many keys (a cache fill): LPK = 8 lanes per key, eight keys per wavefront, 16 columns per
// lane from two 16-byte loads. One key per wavefront spends most of its instructions on work
// done once per key (the sums' exchanges, the square root and division, the scale), with 64
// lanes for 128 values; here that work serves eight keys at once. The LayerNorm sums follow
// insert_key's order, as layer_norm_pair does: 16 running totals of 8 consecutive columns, each
// starting at 0, combined by a butterfly over total offsets 8, 4, 2, 1. Lane `sub` of a key
// holds totals P sub .. P sub + P - 1 (P = 16 / LPK), so an offset of P or more pairs lanes
// sub ^ (offset / P) and a smaller one pairs totals inside the lane. Every operation has the
// same two operands as on one wavefront, so the bytes are the same.
template <int LPK>
__device__ __forceinline__ float bulk_page_sum(const float (&z)[128 / LPK]) {
    constexpr int P = 16 / LPK;  // running totals per lane
    auto add_rn = [](float a, float c) { return __fadd_rn(a, c); };
    float t[P];
#pragma unroll
    for (int m = 0; m < P; ++m) {
        t[m] = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) t[m] = __fadd_rn(t[m], z[8 * m + i]);
    }
#pragma unroll
    for (int m = 0; m < P; ++m) {  // offsets 8, 4, 2 (P = 2) or 8, 4, 2, 1 (P = 1) across lanes
        t[m] = xor_combine<8 / P>(t[m], add_rn);
        t[m] = xor_combine<4 / P>(t[m], add_rn);
        t[m] = xor_combine<2 / P>(t[m], add_rn);
        if constexpr (P == 1) t[m] = xor_combine<1>(t[m], add_rn);
    }
    if constexpr (P == 2) return __fadd_rn(t[0], t[1]);  // offset 1 inside the lane
    else return t[0];
}

// value of lane l + D inside its row of 16 lanes (D < 16 - l % 16)
template <int D>
__device__ __forceinline__ uint32_t row_shl(uint32_t v) {
    return __builtin_amdgcn_update_dpp(0u, v, 0x100 + D, 0xF, 0xF, false);
}

template <int FMT, int LPK>
__global__ __launch_bounds__(256) void store_keys_bulk_kernel(
    const uint16_t *__restrict__ keys, int64_t k_row_stride, int64_t tokens,
    const float *__restrict__ gamma, const float *__restrict__ beta,
    const int64_t *__restrict__ slots, uint8_t *__restrict__ cache, float eps, int64_t num_pages,
    int64_t page_stride) {
    static_assert(LPK == 8 || LPK == 16, "8 or 16 lanes per key");
    constexpr int C = 128 / LPK;  // columns per lane
    const int sub = threadIdx.x & (LPK - 1);  // the lane's place among its key's lanes
    const int64_t t = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPK;
    const int64_t tk = t < tokens ? t : tokens - 1;  // lanes past the end redo the last key
    const uint4 *kr = reinterpret_cast<const uint4 *>(keys + tk * k_row_stride + C * sub);
    const float4 *g4 = reinterpret_cast<const float4 *>(gamma + C * sub);
    const float4 *b4 = reinterpret_cast<const float4 *>(beta + C * sub);
    uint4 raw[C / 8];
    float4 gv[C / 4], bv[C / 4];
#pragma unroll
    for (int i = 0; i < C / 8; ++i) raw[i] = kr[i];
#pragma unroll
    for (int i = 0; i < C / 4; ++i) {
        gv[i] = g4[i];
        bv[i] = b4[i];
    }
    const int64_t slot = slots[tk];
    hoist_args(cache, eps, num_pages, page_stride);
    float x[C], g[C], b[C];
#pragma unroll
    for (int i = 0; i < C / 8; ++i) {
        const uint32_t w[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[8 * i + 2 * k] = bf16_lo(w[k]);
            x[8 * i + 2 * k + 1] = bf16_hi(w[k]);
        }
    }
#pragma unroll
    for (int i = 0; i < C / 4; ++i) {
        g[4 * i] = gv[i].x, g[4 * i + 1] = gv[i].y, g[4 * i + 2] = gv[i].z, g[4 * i + 3] = gv[i].w;
        b[4 * i] = bv[i].x, b[4 * i + 1] = bv[i].y, b[4 * i + 2] = bv[i].z, b[4 * i + 3] = bv[i].w;
    }
    const float mean = __fmul_rn(bulk_page_sum<LPK>(x), 0.0078125f);
    float d[C], sq[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        d[j] = __fsub_rn(x[j], mean);
        sq[j] = __fmul_rn(d[j], d[j]);
    }
    const float var = __fmul_rn(bulk_page_sum<LPK>(sq), 0.0078125f);
    const float rstd = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(var, eps)));
    float n[C];
#pragma unroll
    for (int j = 0; j < C; ++j) n[j] = bf16_round(__fadd_rn(__fmul_rn(__fmul_rn(d[j], rstd), g[j]), b[j]));

    // all lanes of a key leave together (padding slot, or lanes past the end), so the exchanges
    // below only meet lanes of their own key
    if (t >= tokens || slot < 0 || slot >= num_pages * kPageTokens) return;
    uint8_t *sec = cache + (slot >> 6) * page_stride;
    const int off = (int)(slot & 63);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < C; ++j) amax = fmaxf(amax, fabsf(n[j]));
    if constexpr (FMT == kFmtMxfp4) {
        amax = group_max<32 / C>(amax);  // the lanes of one 32-column block
        const int e = ue8m0_exponent(amax);
        const float inv = pow2_neg(e);
        uint32_t word[C / 8];
#pragma unroll
        for (int i = 0; i < C / 8; ++i) {
            uint32_t w = e2m1_pair<0>(0u, __fmul_rn(n[8 * i], inv), __fmul_rn(n[8 * i + 1], inv));
            w = e2m1_pair<1>(w, __fmul_rn(n[8 * i + 2], inv), __fmul_rn(n[8 * i + 3], inv));
            w = e2m1_pair<2>(w, __fmul_rn(n[8 * i + 4], inv), __fmul_rn(n[8 * i + 5], inv));
            w = e2m1_pair<3>(w, __fmul_rn(n[8 * i + 6], inv), __fmul_rn(n[8 * i + 7], inv));
            word[i] = w;
        }
        if constexpr (C == 16)
            *reinterpret_cast<uint2 *>(sec + off * 64 + 8 * sub) = make_uint2(word[0], word[1]);
        else
            *reinterpret_cast<uint32_t *>(sec + off * 64 + 4 * sub) = word[0];
        // block k's exponent sits in the key's lane k * 32 / C; one lane writes the four bytes
        const uint32_t sc = (uint32_t)(e + 127);
        constexpr int B = 32 / C;  // lanes per block
        const uint32_t scales = sc | (row_shl<B>(sc) << 8) | (row_shl<2 * B>(sc) << 16) |
                                (row_shl<3 * B>(sc) << 24);
        if (sub == 0) *reinterpret_cast<uint32_t *>(sec + 64 * 64 + off * 4) = scales;
    } else {
        amax = group_max<LPK>(fmaxf(1e-10f, amax));
        const float s = pow2_ceil(__fdiv_rn(amax, 448.0f));
        const float inv = __fdiv_rn(1.0f, s);
        uint32_t w[C / 4];
#pragma unroll
        for (int i = 0; i < C / 4; ++i)
            w[i] = e4m3x4(__fmul_rn(n[4 * i], inv), __fmul_rn(n[4 * i + 1], inv),
                          __fmul_rn(n[4 * i + 2], inv), __fmul_rn(n[4 * i + 3], inv));
        if constexpr (C == 16)
            *reinterpret_cast<uint4 *>(sec + off * 128 + 16 * sub) = make_uint4(w[0], w[1], w[2], w[3]);
        else
            *reinterpret_cast<uint2 *>(sec + off * 128 + 8 * sub) = make_uint2(w[0], w[1]);
        if (sub == 0) {
            if constexpr (FMT == kFmtFp8Mx)
                *reinterpret_cast<uint32_t *>(sec + 64 * 128 + off * 4) =
                    (__float_as_uint(s) >> 23) * 0x01010101u;
            else
                *reinterpret_cast<float *>(sec + 64 * 128 + off * 4) = s;
        }
    }
}

// The indexer inputs of one step in one launch (page
// "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index", DsaIndex): one workgroup
// per token quantizes the token's query with the head weights read from the packed projection
// row, and normalizes, quantizes and inserts the key held in the same row. With a layout,
// one more workgroup computes the row bounds (decode_layout) in the same launch. `w_in` and
// `key_in` point at the weight and key columns of projection row 0.
// Five wavefronts: four quantize the query, the fifth normalizes, quantizes and inserts the
// key at the same time (with the key on one of the four, its work followed that wavefront's
// share of the query).
constexpr int kInputsThreads = 320;

template <int FMT, int H>
__global__ __launch_bounds__(kInputsThreads) void index_inputs_kernel(
    int64_t tokens, const uint16_t *__restrict__ q, int64_t q_row_stride, int64_t q_head_stride,
    const uint16_t *__restrict__ w_in, int64_t proj_row_stride,
    const uint16_t *__restrict__ key_in, uint8_t *__restrict__ q_out, int64_t q_out_row_stride,
    uint16_t *__restrict__ w_out, int64_t w_out_row_stride, float c_h,
    const float *__restrict__ gamma, const float *__restrict__ beta, float eps,
    const int64_t *__restrict__ slots, uint8_t *__restrict__ cache, int64_t num_pages,
    int64_t page_stride, LayoutArgs layout) {
    const int64_t token = blockIdx.x;
    if (token == tokens) {  // the extra workgroup of the combined call: the row bounds
        decode_layout_body<kInputsThreads>(layout);
        return;
    }
    // uniform across the wavefront, said explicitly so the split below is a scalar branch
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave == 4) {
        const int lane = threadIdx.x & 63;
        hoist_args(gamma, beta, eps, slots, cache, num_pages, page_stride);
        store_key<FMT>(load_key(key_in + token * proj_row_stride, gamma, beta, slots + token, lane),
                       eps, cache, num_pages, page_stride, lane);
        return;
    }
    // the query row and its weights (every operand a preloaded argument), then the other
    // arguments in one batch
    QueryLoads<H> in;
    in.load(q + token * q_row_stride, q_head_stride, threadIdx.x);
    in.load_weights(w_in + token * proj_row_stride, threadIdx.x);
    hoist_args(q_out, q_out_row_stride, w_out, w_out_row_stride, c_h);
    quantize_query_row<FMT, H>(in, true, q_out + token * q_out_row_stride,
                               w_out + token * w_out_row_stride, c_h, threadIdx.x);
}

template <int FMT, int H>
static void launch_quantize_h(dim3 grid, hipStream_t stream, const uint16_t *q,
                              int64_t q_row_stride, int64_t q_head_stride, const uint16_t *wv,
                              int64_t wv_row_stride, uint8_t *q_out, int64_t q_out_row_stride,
                              uint16_t *w_out, int64_t w_out_row_stride, float c_h) {
    hipLaunchKernelGGL((quantize_queries_kernel<FMT, H>), grid, dim3(256), 0, stream, q,
                       q_row_stride, q_head_stride, wv, wv_row_stride, q_out, q_out_row_stride,
                       w_out, w_out_row_stride, c_h);
}

template <int FMT>
static void launch_quantize_fmt(int heads, dim3 grid, hipStream_t stream, const uint16_t *q,
                                int64_t q_row_stride, int64_t q_head_stride, const uint16_t *wv,
                                int64_t wv_row_stride, uint8_t *q_out, int64_t q_out_row_stride,
                                uint16_t *w_out, int64_t w_out_row_stride, float c_h) {
    switch (heads) {
        case 16: return launch_quantize_h<FMT, 16>(grid, stream, q, q_row_stride, q_head_stride, wv,
                                                   wv_row_stride, q_out, q_out_row_stride, w_out,
                                                   w_out_row_stride, c_h);
        case 32: return launch_quantize_h<FMT, 32>(grid, stream, q, q_row_stride, q_head_stride, wv,
                                                   wv_row_stride, q_out, q_out_row_stride, w_out,
                                                   w_out_row_stride, c_h);
        default: return launch_quantize_h<FMT, 64>(grid, stream, q, q_row_stride, q_head_stride, wv,
                                                   wv_row_stride, q_out, q_out_row_stride, w_out,
                                                   w_out_row_stride, c_h);
    }
}

hipError_t launch_quantize_queries(int fmt, const void *q, int64_t rows, int heads,
                                   int64_t q_row_stride, int64_t q_head_stride, const void *wv,
                                   int64_t wv_row_stride, void *q_out, int64_t q_out_row_stride,
                                   void *w_out, int64_t w_out_row_stride, float c_h,
                                   hipStream_t stream) {
    const dim3 grid((unsigned)rows);
    auto *qq = static_cast<const uint16_t *>(q);
    auto *ww = static_cast<const uint16_t *>(wv);
    auto *qo = static_cast<uint8_t *>(q_out);
    auto *wo = static_cast<uint16_t *>(w_out);
    // the FP8 query is the same for both FP8 key layouts
    if (fmt == kFmtMxfp4)
        launch_quantize_fmt<kFmtMxfp4>(heads, grid, stream, qq, q_row_stride, q_head_stride, ww,
                                       wv_row_stride, qo, q_out_row_stride, wo, w_out_row_stride,
                                       c_h);
    else
        launch_quantize_fmt<kFmtFp8>(heads, grid, stream, qq, q_row_stride, q_head_stride, ww,
                                     wv_row_stride, qo, q_out_row_stride, wo, w_out_row_stride,
                                     c_h);
    return hipGetLastError();
}

hipError_t launch_store_keys(int fmt, const void *keys, int64_t tokens, int64_t k_row_stride,
                             const float *gamma, const float *beta, float eps,
                             const int64_t *slots, void *cache, int64_t num_pages,
                             int64_t page_stride, hipStream_t stream) {
    auto *kk = static_cast<const uint16_t *>(keys);
    auto *cc = static_cast<uint8_t *>(cache);
    auto a16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    if (a16(keys) && k_row_stride % 8 == 0 && a16(gamma) && a16(beta)) {
        // 16-byte rows and LayerNorm parameters: eight lanes per key
        constexpr int kLanes = 8;
        const dim3 gridb((unsigned)((tokens * kLanes + 255) / 256)), blockb(256);
        if (fmt == kFmtMxfp4)
            hipLaunchKernelGGL((store_keys_bulk_kernel<kFmtMxfp4, kLanes>), gridb, blockb, 0, stream,
                               kk, k_row_stride, tokens, gamma, beta, slots, cc, eps, num_pages,
                               page_stride);
        else if (fmt == kFmtFp8)
            hipLaunchKernelGGL((store_keys_bulk_kernel<kFmtFp8, kLanes>), gridb, blockb, 0, stream,
                               kk, k_row_stride, tokens, gamma, beta, slots, cc, eps, num_pages,
                               page_stride);
        else
            hipLaunchKernelGGL((store_keys_bulk_kernel<kFmtFp8Mx, kLanes>), gridb, blockb, 0, stream,
                               kk, k_row_stride, tokens, gamma, beta, slots, cc, eps, num_pages,
                               page_stride);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((tokens + 3) / 4)), block(256);
    if (fmt == kFmtMxfp4)
        hipLaunchKernelGGL(store_keys_kernel<kFmtMxfp4>, grid, block, 0, stream, kk, k_row_stride,
                           tokens, gamma, beta, slots, cc, eps, num_pages, page_stride);
    else if (fmt == kFmtFp8)
        hipLaunchKernelGGL(store_keys_kernel<kFmtFp8>, grid, block, 0, stream, kk, k_row_stride,
                           tokens, gamma, beta, slots, cc, eps, num_pages, page_stride);
    else
        hipLaunchKernelGGL(store_keys_kernel<kFmtFp8Mx>, grid, block, 0, stream, kk, k_row_stride,
                           tokens, gamma, beta, slots, cc, eps, num_pages, page_stride);
    return hipGetLastError();
}

struct IndexInputs {
    int64_t tokens;
    const uint16_t *q;
    int64_t q_row_stride, q_head_stride;
    const uint16_t *w_in;
    int64_t proj_row_stride;
    const uint16_t *key_in;
    uint8_t *q_out;
    int64_t q_out_row_stride;
    uint16_t *w_out;
    int64_t w_out_row_stride;
    float c_h;
    const float *gamma, *beta;
    float eps;
    const int64_t *slots;
    uint8_t *cache;
    int64_t num_pages, page_stride;
    LayoutArgs layout;
};

template <int FMT, int H>
static void launch_index_inputs_h(const IndexInputs &a, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((index_inputs_kernel<FMT, H>), grid, dim3(kInputsThreads), 0, stream, a.tokens, a.q,
                       a.q_row_stride, a.q_head_stride, a.w_in, a.proj_row_stride, a.key_in,
                       a.q_out, a.q_out_row_stride, a.w_out, a.w_out_row_stride, a.c_h, a.gamma,
                       a.beta, a.eps, a.slots, a.cache, a.num_pages, a.page_stride, a.layout);
}

template <int FMT>
static void launch_index_inputs_fmt(int heads, const IndexInputs &a, dim3 grid,
                                    hipStream_t stream) {
    switch (heads) {
        case 16: return launch_index_inputs_h<FMT, 16>(a, grid, stream);
        case 32: return launch_index_inputs_h<FMT, 32>(a, grid, stream);
        default: return launch_index_inputs_h<FMT, 64>(a, grid, stream);
    }
}

hipError_t launch_index_inputs(int fmt, const void *projected, int64_t tokens,
                               int64_t proj_row_stride, int64_t key_col, int64_t weight_col,
                               const void *q, int heads, int64_t q_row_stride,
                               int64_t q_head_stride, const float *gamma, const float *beta,
                               float eps, const int64_t *slots, void *cache, int64_t num_pages,
                               int64_t page_stride, void *q_out, int64_t q_out_row_stride,
                               void *w_out, int64_t w_out_row_stride, float c_h,
                               const LayoutArgs *layout, hipStream_t stream) {
    const dim3 grid((unsigned)(tokens + (layout ? 1 : 0)));
    auto *pp = static_cast<const uint16_t *>(projected);
    const IndexInputs a{tokens, static_cast<const uint16_t *>(q), q_row_stride, q_head_stride,
                        pp + weight_col, proj_row_stride, pp + key_col,
                        static_cast<uint8_t *>(q_out), q_out_row_stride,
                        static_cast<uint16_t *>(w_out), w_out_row_stride, c_h, gamma, beta, eps,
                        slots, static_cast<uint8_t *>(cache), num_pages, page_stride,
                        layout ? *layout : LayoutArgs{}};
    if (fmt == kFmtMxfp4) launch_index_inputs_fmt<kFmtMxfp4>(heads, a, grid, stream);
    else if (fmt == kFmtFp8) launch_index_inputs_fmt<kFmtFp8>(heads, a, grid, stream);
    else launch_index_inputs_fmt<kFmtFp8Mx>(heads, a, grid, stream);
    return hipGetLastError();
}

}  // namespace dsaidx
