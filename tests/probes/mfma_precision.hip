// Test probe (not part of the library): dot products through the gfx950 scaled FP8 matrix
// instruction (E4M3 x E4M3, unit block scales) and through the BF16 matrix instruction, so that
// a test can compare their rounding with the exact sums. The FP8 scoring path relies on the
// second (E4M3 widened exactly to BF16); the first keeps too few bits below a block's largest
// product for the logit tolerance.
//
// One wavefront computes one 16 x 16 tile over K = 128. Both operands are given as the bytes each
// lane holds (A and B in the same per-lane form), so element (i, j) pairs A's and B's values at
// the same place of the same lane group whatever the instruction's lane layout: with every lane
// holding the same pattern, each element is 4 times the pattern's dot product (FP8: 32 values per
// lane, one instruction; BF16: 8 values per lane and instruction, four chained instructions over
// the same 32 values).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// a, b: 32 bytes per lane (E4M3), lane l at bytes [32 l, 32 l + 32); out: 4 floats per lane
__global__ void fp8_scaled_tile(const int *a, const int *b, float *out) {
    const int l = threadIdx.x;
    v8i va, vb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        va[i] = a[8 * l + i];
        vb[i] = b[8 * l + i];
    }
    v4f c = {0.f, 0.f, 0.f, 0.f};
    // format 0 = E4M3 for both operands; block scales 127 (2^0) in byte 0
    c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, c, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[4 * l + i] = c[i];
}

// a, b: 64 bytes per lane (32 BF16), lane l at bytes [64 l, 64 l + 64): instruction kk takes
// the lane's values 8 kk .. 8 kk + 7
__global__ void bf16_tile(const int *a, const int *b, float *out) {
    const int l = threadIdx.x;
    v4f c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        int ra[4], rb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = a[16 * l + 4 * kk + i];
            rb[i] = b[16 * l + 4 * kk + i];
        }
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, ra),
                                                   __builtin_bit_cast(v8bf, rb), c, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) out[4 * l + i] = c[i];
}

// Device pointers: fp8 a, b of 2048 bytes; bf16 a, b of 4096 bytes; out of 256 floats.
// Runs on the null stream and waits; returns the HIP status.
extern "C" int probe_fp8_scaled_tile(const void *a, const void *b, float *out) {
    hipLaunchKernelGGL(fp8_scaled_tile, dim3(1), dim3(64), 0, 0, static_cast<const int *>(a),
                       static_cast<const int *>(b), out);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}

extern "C" int probe_bf16_tile(const void *a, const void *b, float *out) {
    hipLaunchKernelGGL(bf16_tile, dim3(1), dim3(64), 0, 0, static_cast<const int *>(a),
                       static_cast<const int *>(b), out);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? (int)e : (int)hipDeviceSynchronize();
}
