// Device helpers of the gfx950 indexer kernels: BF16 conversion, the E2M1 / E4M3 encoders,
// UE8M0 and power-of-two scale exponents from FP32 bit fields, and wavefront reductions.
//
// Format definitions: page "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index"
// (module text: MXFP4 = one UE8M0 scale per 32 values, E2M1 round to nearest even with
// saturation; e2m1x2; mxfp4_scale; DsaIndex.fp8_query).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsaidx {

constexpr int kDim = 128;
constexpr int kPageTokens = 64;
constexpr int kMxfp4Section = 64 * 64 + 64 * 4;   // 4352
constexpr int kFp8Section = 64 * 128 + 64 * 4;    // 8448
constexpr int kFmtMxfp4 = 0;
constexpr int kFmtFp8 = 1;
constexpr int kFmtFp8Mx = 2;  // FP8 keys, scale stored as four equal UE8M0 bytes
constexpr bool is_fp8(int fmt) { return fmt != kFmtMxfp4; }

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_val(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
    uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float(bf16_bits_rne(f) << 16); }

// Two E2M1 codes, of a (low nibble) and b (high nibble), into byte `Byte` of `word` (the
// other bytes kept), by the gfx950 scaled conversion with scale 1. The code of a value is its
// nearest point of the grid 0, .5, 1, 1.5, 2, 3, 4, 6 (ties to the even code: 0.25 -> 0,
// 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4), magnitudes above 5 saturate
// to 6, and bit 3 is the input's sign bit (so -0 gives 8). A probe on the device compared
// the instruction with these comparisons written out over the grid, every midpoint, their
// FP32 neighbours, both signs, subnormals, huge values and 200,000 random values in [-7, 7]:
// no difference.
template <int Byte>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t word, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, a, b, 1.0f, Byte);
}

// The E2M1 codes of the two BF16 values packed in `pair` (low half -> low nibble) times 2^-e,
// e in [-126, 126], into byte Byte of `word`: the gfx950 BF16 scaled conversion with scale
// 2^e, which divides by its scale. A probe on the device compared it with e2m1_pair of the
// exact FP32 products for every finite BF16 pattern (and its negation) at every such e: no
// difference.
template <int Byte>
__device__ __forceinline__ uint32_t e2m1_bf16_pair(uint32_t word, uint32_t pair, int e) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const float scale = __uint_as_float((uint32_t)(127 + e) << 23);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, __builtin_bit_cast(bf16x2, pair), scale,
                                                     Byte);
}

// E4M3FN codes of values already scaled into [-448, 448] (every quantizer here divides by a
// power-of-two scale no smaller than amax / 448, so nothing reaches the saturating branch):
// the gfx950 conversion, which rounds to nearest even, subnormals (units of 2^-9) included,
// and keeps the sign of values that round to zero (code 0x80). A device probe compared it with
// the rounding written out in integer arithmetic (the FP32 mantissa rounded to 3 bits with its
// carry into the exponent, rebiased 127 -> 7; below 2^-6 the value in units of 2^-9, nearest
// even) on 1.67 M values: every FP32 pattern's top 20 bits up to 448 with random low bits, the
// E4M3 grid, its midpoints and their FP32 neighbours, both signs: no difference.
// e4m3x2: two codes (a low byte, b next); e4m3x4: four (a lowest).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// UE8M0 exponent e of an MXFP4 block: the smallest integer with 6 * 2^e >= max(amax,
// 6 * 2^-126). For amax = M * 2^E (M in [1, 2)) that is E - 2 when M <= 1.5 and E - 1 when
// M > 1.5; every amax below 6 * 2^-126 (bits 0x01C00000) gives -126.
__device__ __forceinline__ int ue8m0_exponent(float amax) {
    const uint32_t b = __float_as_uint(amax);
    if (b < 0x01C00000u) return -126;
    return (int)(b >> 23) - 129 + ((b & 0x7FFFFFu) > 0x400000u ? 1 : 0);
}

// 2^-e for e in [-126, 126], built from its exponent field.
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// Smallest power of two >= x (x positive and normal).
__device__ __forceinline__ float pow2_ceil(float x) {
    uint32_t b = __float_as_uint(x);
    if (b & 0x7FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;
    return __uint_as_float(b);
}

// Correctly rounded FP32 square root of a positive normal value. The hardware estimate y is
// within one ulp, so the answer is y or a neighbour y' = y -+ 1 ulp. For neighbours a < b the
// midpoint satisfies mid^2 = a*b + (b - a)^2 / 4, and x - a*b is an exact multiple of
// (b - a)^2 (both x and a*b are), so sqrt(x) < mid exactly when x - a*b <= 0. One fused
// multiply-add gives the sign of x - a*b exactly, which picks the rounding.
__device__ __forceinline__ float sqrt_rn(float x) {
    float y = __builtin_amdgcn_sqrtf(x);
    const float below = __uint_as_float(__float_as_uint(y) - 1u);
    const float above = __uint_as_float(__float_as_uint(y) + 1u);
    if (__builtin_fmaf(-below, y, x) <= 0.0f) y = below;
    else if (__builtin_fmaf(-y, above, x) > 0.0f) y = above;
    return y;
}

// Cross-lane exchanges in registers: DPP for partners inside a row of 16 lanes, the gfx950
// lane swaps across rows (an LDS permute costs a round trip through the LDS unit instead).
// lane_xor<H>(v), H = 1, 2, 4, 8: the value of lane l ^ H.
template <int H>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    static_assert(H == 1 || H == 2 || H == 4 || H == 8, "partner inside a row of 16 lanes");
    if constexpr (H == 1) {
        return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    } else if constexpr (H == 2) {
        return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    } else if constexpr (H == 4) {
        const uint32_t up = __builtin_amdgcn_update_dpp(0u, v, 0x104, 0xF, 0xF, false);  // row_shl:4: i + 4
        const uint32_t dn = __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);  // row_shr:4: i - 4
        return (threadIdx.x & 4) ? dn : up;
    } else {
        return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xF, 0xF, false);  // row_ror:8: i ^ 8
    }
}

// op(v, v of lane l ^ H) in every lane, H = 1 .. 32; `op` commutative, so the result is
// exactly op(own, partner) whichever operand order the lane swaps deliver.
template <int H, typename T, typename Op>
__device__ __forceinline__ T xor_combine(T v, Op op) {
    static_assert(sizeof(T) == 4, "32-bit values");
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    if constexpr (H <= 8) {
        return op(v, __builtin_bit_cast(T, lane_xor<H>(u)));
    } else if constexpr (H == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows 0<->1, 2<->3
        return op(__builtin_bit_cast(T, (uint32_t)r[0]), __builtin_bit_cast(T, (uint32_t)r[1]));
    } else {
        static_assert(H == 32, "H = 1 .. 32");
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // halves
        return op(__builtin_bit_cast(T, (uint32_t)r[0]), __builtin_bit_cast(T, (uint32_t)r[1]));
    }
}

__device__ __forceinline__ float max_of(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ int max_of(int a, int b) { return max(a, b); }

// max over each aligned group of LANES lanes (a power of two up to 64), in all of them (fmaxf
// for floats: a NaN operand gives the other one)
template <int LANES, typename T>
__device__ __forceinline__ T group_max(T v) {
    auto mx = [](T a, T b) { return max_of(a, b); };
    if constexpr (LANES > 1) v = xor_combine<1>(v, mx);
    if constexpr (LANES > 2) v = xor_combine<2>(v, mx);
    if constexpr (LANES > 4) v = xor_combine<4>(v, mx);
    if constexpr (LANES > 8) v = xor_combine<8>(v, mx);
    if constexpr (LANES > 16) v = xor_combine<16>(v, mx);
    if constexpr (LANES > 32) v = xor_combine<32>(v, mx);
    return v;
}

// value of lane l + D (D = 1, 2, 3) inside each quad of lanes, for lane l % 4 == 0 (other
// lanes get a value of no use)
template <int D>
__device__ __forceinline__ uint32_t quad_down(uint32_t v) {
    static_assert(D >= 1 && D <= 3, "inside a quad");
    // quad_perm selectors: lane 0 <- D, lanes 1..3 <- min(lane + D, 3)
    constexpr int c = D == 1 ? 0xF9 : D == 2 ? 0xFE : 0xFF;
    return __builtin_amdgcn_update_dpp(0u, v, c, 0xF, 0xF, false);
}

// value of lane 4 * (l / 4) + I (lane I of l's quad), in every lane
template <int I>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
    static_assert(I >= 0 && I <= 3, "inside a quad");
    return __builtin_amdgcn_update_dpp(0u, v, I * 0x55, 0xF, 0xF, false);  // quad_perm [I,I,I,I]
}

// value of lane l + D (D = 4, 8, 12) inside each row of 16 lanes, for lane l % 16 == 0
template <int D>
__device__ __forceinline__ uint32_t row_down(uint32_t v) {
    static_assert(D == 4 || D == 8 || D == 12, "inside a row of 16");
    return __builtin_amdgcn_update_dpp(0u, v, 0x100 + D, 0xF, 0xF, false);  // row_shl:D
}

// Kernel arguments are read from memory, and the compiler loads each one next to its first use;
// in a short kernel those loads form a chain of round trips, each waited for before the next
// is issued. Naming the arguments here, at the kernel's entry, loads all of them at once.
template <typename T>
__device__ __forceinline__ void hoist_arg(const T &v) {
    asm volatile("" ::"s"(v));
}
template <typename... T>
__device__ __forceinline__ void hoist_args(const T &...v) {
    (hoist_arg(v), ...);
}

// A use of a loaded value that emits nothing. The compiler moves a load down into the one
// branch that uses its value, which would put a load issued early on purpose behind the
// checks it is meant to overlap; a use on the other branch as well keeps it where it is
// written. The use waits for the load, so it belongs on a branch that does nothing else
// (an early return).
__device__ __forceinline__ void keep_loaded(uint32_t v) { asm volatile("" ::"v"(v)); }

// Waits for every vector memory operation in flight, so that no later instruction does: placed
// after a batch of loads and before any store, it keeps the compiler from waiting on a register
// a load might still write at a point where stores are in flight too -- one counter counts both,
// so every such use after a store would wait for the stores as well.
__device__ __forceinline__ void loads_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Order-preserving 32-bit key of a logit for the top-k selection: unsigned comparison of
// keys is the float order, with -0 mapped to +0 so the two compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t b = __float_as_uint(f);
    if (b == 0x80000000u) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

}  // namespace dsaidx
