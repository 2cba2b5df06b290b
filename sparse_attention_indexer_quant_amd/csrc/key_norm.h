// The key path shared by the key-insert kernels and the scorer that inserts a step's keys
// itself: LayerNorm of one 128-value BF16 key on one wavefront (FP32, then rounded to BF16)
// and its MXFP4 encoding.
//
// Page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index", insert_key and
// insert_fp4_key: the key is LayerNorm(wk projection) in FP32, then BF16, then quantized; the
// MXFP4 section holds the 64 B payload at token * 64 and the four UE8M0 bytes at
// 64 * 64 + token * 4.
#pragma once

#include "device_common.h"

namespace dsaidx {

// One key's inputs as one lane of its wavefront holds them: columns 2l and 2l+1 (one 4-byte
// load), their LayerNorm weights and biases, and the key's slot.
struct KeyLane {
    uint32_t pair;
    float2 g, b;
    int64_t slot;
};

__device__ __forceinline__ KeyLane load_key(const uint16_t *__restrict__ key,
                                            const float *__restrict__ gamma,
                                            const float *__restrict__ beta,
                                            const int64_t *__restrict__ slot, int lane) {
    KeyLane k;
    k.pair = *reinterpret_cast<const uint32_t *>(key + 2 * lane);
    k.g = *reinterpret_cast<const float2 *>(gamma + 2 * lane);
    k.b = *reinterpret_cast<const float2 *>(beta + 2 * lane);
    k.slot = slot ? *slot : 0;
    return k;
}

// Sum of the key's 128 values in the order insert_key uses: 16 running totals, total j adding
// columns 8j .. 8j+7 one at a time to 0, then the totals combined by a butterfly over total
// offsets 8, 4, 2, 1 (the page hides that combine; read as the order of its group_max). Here
// total j is formed, the same in every lane, by the quad of lanes 4j .. 4j+3 (which hold its
// columns two per lane), so the butterfly's total offsets are lane offsets 32, 16, 8, 4.
// `v` holds the quad's eight values in column order.
__device__ __forceinline__ float page_order_sum(const float (&v)[8]) {
    auto add_rn = [](float a, float b) { return __fadd_rn(a, b); };
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t = __fadd_rn(t, v[i]);
    t = xor_combine<32>(t, add_rn);
    t = xor_combine<16>(t, add_rn);
    t = xor_combine<8>(t, add_rn);
    t = xor_combine<4>(t, add_rn);
    return t;
}

// The lane's two LayerNorm outputs (columns 2l, 2l+1), rounded to BF16: mean = S(x) / 128,
// variance = S((x - mean) * (x - mean)) / 128 with each square rounded before it is added,
// rstd = 1 / sqrt(variance + eps) (IEEE square root, then IEEE divide), y = ((x - mean) *
// rstd) * gamma + beta, every step one RN operation.
__device__ __forceinline__ void layer_norm_pair(const KeyLane &in, float eps, float &n0,
                                                float &n1) {
    const float x0 = bf16_lo(in.pair), x1 = bf16_hi(in.pair);
    float v[8];  // columns 8 (l / 4) .. 8 (l / 4) + 7: the pairs of the lane's quad
    const uint32_t q0 = quad_bcast<0>(in.pair), q1 = quad_bcast<1>(in.pair),
                   q2 = quad_bcast<2>(in.pair), q3 = quad_bcast<3>(in.pair);
    v[0] = bf16_lo(q0), v[1] = bf16_hi(q0), v[2] = bf16_lo(q1), v[3] = bf16_hi(q1);
    v[4] = bf16_lo(q2), v[5] = bf16_hi(q2), v[6] = bf16_lo(q3), v[7] = bf16_hi(q3);
    const float mean = __fmul_rn(page_order_sum(v), 0.0078125f);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float d = __fsub_rn(v[i], mean);
        v[i] = __fmul_rn(d, d);
    }
    const float var = __fmul_rn(page_order_sum(v), 0.0078125f);
    const float rstd = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(var, eps)));
    const float d0 = __fsub_rn(x0, mean), d1 = __fsub_rn(x1, mean);
    n0 = bf16_round(__fadd_rn(__fmul_rn(__fmul_rn(d0, rstd), in.g.x), in.b.x));
    n1 = bf16_round(__fadd_rn(__fmul_rn(__fmul_rn(d1, rstd), in.g.y), in.b.y));
}

// The lane's MXFP4 payload byte (columns 2l, 2l+1: byte l of the token's 64) and the UE8M0
// byte of its 32-column block (block l / 16; the 16 lanes of a block hold the same value).
struct Mxfp4KeyLane {
    uint32_t byte;
    uint32_t scale;
};

__device__ __forceinline__ Mxfp4KeyLane mxfp4_key_lane(float n0, float n1) {
    const float amax = group_max<16>(fmaxf(fabsf(n0), fabsf(n1)));  // 16 lanes = 32 columns
    const int e = ue8m0_exponent(amax);
    const float inv = pow2_neg(e);
    return {e2m1_pair<0>(0u, __fmul_rn(n0, inv), __fmul_rn(n1, inv)) & 0xFFu, (uint32_t)(e + 127)};
}

// Writes the key to token `off` of the MXFP4 section `sec`.
__device__ __forceinline__ void store_mxfp4_key(const Mxfp4KeyLane &k, uint8_t *sec, int off,
                                                int lane) {
    const uint32_t word = k.byte | (quad_down<1>(k.byte) << 8) | (quad_down<2>(k.byte) << 16) |
                          (quad_down<3>(k.byte) << 24);
    if ((lane & 3) == 0) *reinterpret_cast<uint32_t *>(sec + off * 64 + lane) = word;
    const uint32_t scales = k.scale | (__builtin_amdgcn_readlane(k.scale, 16) << 8) |
                            (__builtin_amdgcn_readlane(k.scale, 32) << 16) |
                            (__builtin_amdgcn_readlane(k.scale, 48) << 24);
    if (lane == 0) *reinterpret_cast<uint32_t *>(sec + 64 * 64 + off * 4) = scales;
}

// The lane's two E4M3 codes (columns 2l, 2l+1, low byte first) and the key's power-of-two
// scale s = pow2_ceil(max(1e-10, amax) / 448) (insert_key's FP8 writer).
struct Fp8KeyLane {
    uint32_t two;
    float s;
};

__device__ __forceinline__ Fp8KeyLane fp8_key_lane(float n0, float n1) {
    const float amax = group_max<64>(fmaxf(1e-10f, fmaxf(fabsf(n0), fabsf(n1))));
    const float s = pow2_ceil(__fdiv_rn(amax, 448.0f));
    const float inv = __fdiv_rn(1.0f, s);
    return {e4m3x2(__fmul_rn(n0, inv), __fmul_rn(n1, inv)), s};
}

// The 4-byte scale word of an FP8 section row: the FP32 scale, or with mx its exponent field
// (s = 2^e is a normal FP32, 2^-42 <= s <= 2^120: the field is e + 127) as four equal bytes.
template <int FMT>
__device__ __forceinline__ uint32_t fp8_scale_word(float s) {
    if constexpr (FMT == kFmtFp8Mx) return (__float_as_uint(s) >> 23) * 0x01010101u;
    else return __float_as_uint(s);
}

// Writes the key to token `off` of the FP8 section `sec`: 128 code bytes, then the scale word.
template <int FMT>
__device__ __forceinline__ void store_fp8_key(const Fp8KeyLane &k, uint8_t *sec, int off, int lane) {
    const uint32_t word = k.two | (quad_down<1>(k.two) << 16);
    if ((lane & 1) == 0) *reinterpret_cast<uint32_t *>(sec + off * 128 + 2 * lane) = word;
    if (lane == 0) *reinterpret_cast<uint32_t *>(sec + 64 * 128 + off * 4) = fp8_scale_word<FMT>(k.s);
}

}  // namespace dsaidx
