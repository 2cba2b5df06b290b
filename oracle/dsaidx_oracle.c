/*
 * CPU oracle of the DSA lightning-indexer hot path (MXFP4 / FP8).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this library. The HIP product path never calls it and
 * shares no code, header, table or constant with it.
 *
 * Every function is written from the definitions on the source pages, in the
 * plainest form: formats are decoded from tables, encoders search those tables
 * for the nearest value, exponents are found by counting, scores are exact
 * integer sums scaled in double precision. Nothing is blocked, fused or
 * reordered. Build with  gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp
 * so that every float operation is one IEEE single-precision operation with
 * round-to-nearest-even, exactly as written.
 *
 * Page citations:
 *   [idx]    vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.index
 *   [fp4ops] vllm.models.kimi_k3.amd.ops.fp4_indexer
 *   [ovl]    vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.dsa.overlap
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_FMT_MXFP4 0
#define ORC_FMT_FP8 1
#define ORC_FMT_FP8_MX 2   /* FP8 keys whose power-of-two scale is stored as UE8M0 bytes */

static int valid_fmt(int fmt) {
    return fmt == ORC_FMT_MXFP4 || fmt == ORC_FMT_FP8 || fmt == ORC_FMT_FP8_MX;
}

#define ORC_OK 0
#define ORC_EINVAL 1

#define DIM 128          /* indexer head / key width: 128 values */
#define PAGE_TOKENS 64   /* tokens per cache page */

/* ------------------------------------------------------------------------ */
/* Scalar formats                                                           */
/* ------------------------------------------------------------------------ */

/* E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit, no Inf/NaN):
 * the sixteen values by code. [idx] e2m1x2 and the module text name the
 * format; the value set is the OCP MX E2M1 definition. */
static const double E2M1_TABLE[16] = {
    0.0,  0.5,  1.0,  1.5,  2.0,  3.0,  4.0,  6.0,
    -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0};

double orc_e2m1_value(int code) { return E2M1_TABLE[code & 15]; }

/* Nearest E2M1 code of an FP32 value, round to nearest with ties to the even
 * code, saturating to +-6 ("round to nearest even, satfinite", [idx] e2m1x2).
 * The sign bit follows the input's sign, also when the result is zero. */
int orc_e2m1_encode(float s) {
    double m = fabs((double)s);
    int best = 7;
    if (m < 6.0) {
        double best_d = INFINITY;
        for (int c = 0; c < 8; ++c) {
            double d = fabs(m - E2M1_TABLE[c]);
            if (d < best_d || (d == best_d && (c & 1) == 0)) {
                best_d = d;
                best = c;
            }
        }
    }
    return best | (signbit(s) ? 8 : 0);
}

/* E4M3FN (bias 7, subnormal step 2^-9, largest finite 448, codes 0x7F/0xFF
 * NaN). The 448 of [idx] DsaIndex.fp8_query fixes the FN variant. The table
 * is filled from the field definition on first use. */
static double E4M3_TABLE[256];
static int e4m3_ready = 0;

static void e4m3_fill(void) {
    for (int c = 0; c < 256; ++c) {
        int sgn = c >> 7, ex = (c >> 3) & 15, man = c & 7;
        double mag;
        if (ex == 15 && man == 7)
            mag = NAN;
        else if (ex == 0)
            mag = ldexp((double)man, -9);
        else
            mag = ldexp((double)(8 + man), ex - 10);
        E4M3_TABLE[c] = sgn ? -mag : mag;
    }
    e4m3_ready = 1;
}

double orc_e4m3_value(int code) {
    if (!e4m3_ready) e4m3_fill();
    return E4M3_TABLE[code & 255];
}

/* Nearest finite E4M3FN code, ties to the even code, saturating at 448
 * (every magnitude >= 448 gives 448: between 448 and the tie at 464 it is the
 * nearest value, above that the saturation). Sign kept on zero results. */
int orc_e4m3_encode(float s) {
    if (!e4m3_ready) e4m3_fill();
    double m = fabs((double)s);
    int best = 0x7E;
    if (m < 448.0) {
        double best_d = INFINITY;
        for (int c = 0; c <= 0x7E; ++c) {
            double d = fabs(m - E4M3_TABLE[c]);
            if (d < best_d || (d == best_d && (c & 1) == 0)) {
                best_d = d;
                best = c;
            }
        }
    }
    return best | (signbit(s) ? 0x80 : 0);
}

/* BF16 round-to-nearest-even of an FP32 value: of the two BF16 neighbours
 * (truncated towards zero, and one BF16 step further out), the nearer one,
 * ties to the even mantissa. */
float orc_bf16_round(float x) {
    uint32_t b;
    memcpy(&b, &x, 4);
    uint32_t lo = b & 0xFFFF0000u, hi = lo + 0x10000u;
    if (lo == b) return x;
    float flo, fhi;
    memcpy(&flo, &lo, 4);
    memcpy(&fhi, &hi, 4);
    double dlo = fabs((double)x - (double)flo), dhi = fabs((double)fhi - (double)x);
    if (dlo < dhi) return flo;
    if (dhi < dlo) return fhi;
    return ((lo >> 16) & 1u) ? fhi : flo;
}

static float bf16_to_f32(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return f;
}

static uint16_t f32_to_bf16_bits(float x) {
    float r = orc_bf16_round(x);
    uint32_t b;
    memcpy(&b, &r, 4);
    return (uint16_t)(b >> 16);
}

/* UE8M0 scale exponent of an MXFP4 block with absolute maximum amax
 * ([idx] mxfp4_scale): scale = 2^clamp(ceil(log2(max(amax, 6*2^-126) / 6)),
 * -127, 127). Read exactly: the smallest integer e with
 * 6 * 2^e >= max(amax, 6 * 2^-126), found by counting up from a lower bound. */
int orc_ue8m0_exponent(float amax) {
    const double lowest = ldexp(6.0, -126);
    double t = (double)amax;
    if (!(t >= lowest)) t = lowest;
    int x;
    frexp(t, &x);  /* t = f * 2^x, f in [0.5, 1) */
    int e = x - 4; /* 6 * 2^(x-4) = 0.375 * 2^x < t: a lower bound */
    while (ldexp(6.0, e) < t) ++e;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

int orc_ue8m0_byte(float amax) { return orc_ue8m0_exponent(amax) + 127; }

/* Smallest power of two >= x, for positive normal x ([idx]
 * DsaIndex.fp8_query takes pow2_ceil of amax / 448). */
float orc_pow2_ceil(float x) {
    int xe;
    frexp((double)x, &xe);
    int e = xe - 2; /* 2^(xe-2) < 0.5 * 2^xe <= x */
    while (ldexp(1.0, e) < (double)x) ++e;
    return (float)ldexp(1.0, e);
}

/* Head-weight factor (heads * 128)^-0.5 in FP32 ([idx] DsaIndex.fp8_query
 * folds the weight with it; the MXFP4 path takes only this indexer weight
 * scale). 2^-6 at 32 heads. */
float orc_head_weight_scale(int heads) {
    return (float)(1.0 / sqrt((double)heads * (double)DIM));
}

/* ------------------------------------------------------------------------ */
/* Key LayerNorm ([idx] insert_key)                                         */
/* ------------------------------------------------------------------------ */

/* Sum of 128 FP32 values in the order [idx] insert_key shows: lane j of a
 * half-warp holds columns 8j .. 8j+7 and adds them one by one to a running
 * total that starts at 0; the sixteen lane totals are then combined by
 * half_warp_sum, whose body the page does not print. It is read here as a
 * butterfly over lane offsets 8, 4, 2, 1 (the descending order of the page's
 * group_max): at each offset o every total t_j becomes t_j + t_(j xor o), and
 * after the four steps every lane holds the same sum. */
float orc_ln_sum128(const float *z) {
    float t[16];
    for (int j = 0; j < 16; ++j) {
        float total = 0.0f;
        for (int i = 0; i < 8; ++i) total += z[8 * j + i];
        t[j] = total;
    }
    for (int o = 8; o >= 1; o /= 2) {
        float next[16];
        for (int j = 0; j < 16; ++j) next[j] = t[j] + t[j ^ o];
        memcpy(t, next, sizeof t);
    }
    return t[0];
}

/* LayerNorm in FP32 of one 128-value key, then rounded to BF16 and widened
 * back to FP32 ([idx] insert_key): mean = sum(x) / 128 and
 * variance = sum((x - mean) * (x - mean)) / 128, both sums in the order of
 * orc_ln_sum128, each square rounded before it is added (no fused multiply-
 * add); rstd = 1 / sqrt(var + eps) (IEEE square root, then IEEE divide: the
 * page's non-fast rsqrt is read as this); y = ((x - mean) * rstd) * gamma + beta
 * with every operation rounded on its own. */
void orc_layernorm128(const float *x, const float *gamma, const float *beta, float eps,
                      float *out) {
    float d[DIM], sq[DIM];
    float mean = orc_ln_sum128(x) / 128.0f;
    for (int i = 0; i < DIM; ++i) {
        d[i] = x[i] - mean;
        sq[i] = d[i] * d[i];
    }
    float var = orc_ln_sum128(sq) / 128.0f;
    float denom = sqrtf(var + eps);
    float rstd = 1.0f / denom;
    for (int i = 0; i < DIM; ++i) {
        float y = d[i] * rstd;
        y = y * gamma[i];
        y = y + beta[i];
        out[i] = orc_bf16_round(y);
    }
}

/* ------------------------------------------------------------------------ */
/* MXFP4 / FP8 of one 128-value vector                                      */
/* ------------------------------------------------------------------------ */

/* MXFP4 of 128 values: four blocks of 32 consecutive values, each with its
 * UE8M0 byte; value v of block g becomes E2M1(v * 2^-e_g) (the page multiplies
 * by 1/scale, exact for a power of two). payload[j] holds columns 2j (low
 * nibble) and 2j+1 (high nibble); scales[g] is block g's byte. */
static void mxfp4_of_128(const float *v, uint8_t *payload, uint8_t *scales) {
    for (int g = 0; g < 4; ++g) {
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[32 * g + i]));
        int e = orc_ue8m0_exponent(amax);
        float inverse = ldexpf(1.0f, -e);
        for (int j = 0; j < 16; ++j) {
            int col = 32 * g + 2 * j;
            int lo = orc_e2m1_encode(v[col] * inverse);
            int hi = orc_e2m1_encode(v[col + 1] * inverse);
            payload[16 * g + j] = (uint8_t)(lo | (hi << 4));
        }
        scales[g] = (uint8_t)(e + 127);
    }
}

/* FP8 with one power-of-two scale for 128 values: amax floored at
 * FP32(1e-10), s = pow2_ceil(amax / 448), value E4M3(v * (1 / s)).
 * Returns s. */
static float fp8_of_128(const float *v, uint8_t *payload) {
    float amax = 1e-10f;
    for (int i = 0; i < DIM; ++i) amax = fmaxf(amax, fabsf(v[i]));
    float s = orc_pow2_ceil(amax / 448.0f);
    float inverse = 1.0f / s;
    for (int i = 0; i < DIM; ++i) payload[i] = (uint8_t)orc_e4m3_encode(v[i] * inverse);
    return s;
}

/* ------------------------------------------------------------------------ */
/* quantize_queries ([idx] quantize_fp4_query, DsaIndex.fp8_query;          */
/* [fp4ops] quantize_queries)                                               */
/* ------------------------------------------------------------------------ */

/* q: BF16 [rows, heads, 128] with element strides; wv: raw BF16 head weights
 * [rows, heads] or NULL. MXFP4 output row: [heads x 64 B E2M1 | heads x 4 B
 * UE8M0], w_out = BF16(wv * c_H). FP8 output row: [heads x 128 B E4M3],
 * w_out = BF16((wv * s_h) * c_H). */
int orc_quantize_queries(int fmt, const uint16_t *q, int64_t rows, int heads,
                         int64_t q_row_stride, int64_t q_head_stride, const uint16_t *wv,
                         int64_t wv_row_stride, uint8_t *q_out, int64_t q_out_row_stride,
                         uint16_t *w_out, int64_t w_out_row_stride) {
    if (!valid_fmt(fmt) || rows < 0 || heads < 1) return ORC_EINVAL;
    const float c_h = orc_head_weight_scale(heads);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        uint8_t *row = q_out + r * q_out_row_stride;
        for (int h = 0; h < heads; ++h) {
            float v[DIM];
            const uint16_t *src = q + r * q_row_stride + (int64_t)h * q_head_stride;
            for (int i = 0; i < DIM; ++i) v[i] = bf16_to_f32(src[i]);
            float w = wv ? bf16_to_f32(wv[r * wv_row_stride + h]) : 0.0f;
            float folded;
            if (fmt == ORC_FMT_MXFP4) {
                mxfp4_of_128(v, row + (int64_t)h * 64, row + (int64_t)heads * 64 + h * 4);
                folded = w * c_h;
            } else {
                float s = fp8_of_128(v, row + (int64_t)h * DIM);
                folded = (w * s) * c_h;
            }
            if (wv && w_out) w_out[r * w_out_row_stride + h] = f32_to_bf16_bits(folded);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* store_keys ([idx] insert_key, insert_fp4_key; [fp4ops] store_keys,       */
/* cache_views)                                                             */
/* ------------------------------------------------------------------------ */

/* Per token: LayerNorm of the BF16 pre-norm key, BF16, then MXFP4 into the
 * 4352-byte section [64 x 64 B E2M1 | 64 x 4 B UE8M0] of page slot / 64 at
 * token offset slot % 64, or FP8 into the 8448-byte section
 * [64 x 128 B E4M3 | 64 x 4 B scale]: the FP32 scale, or for FP8_MX the
 * scale's exponent e (the scale is 2^e) as four equal UE8M0 bytes e + 127
 * ([idx] module text and insert_key, mx). Section p starts at
 * cache + p * page_stride. A negative slot is padding and writes nothing;
 * a slot at or beyond num_pages * 64 writes nothing either. */
int orc_store_keys(int fmt, const uint16_t *keys, int64_t tokens, int64_t k_row_stride,
                   const float *gamma, const float *beta, float eps, const int64_t *slots,
                   uint8_t *cache, int64_t num_pages, int64_t page_stride) {
    if (!valid_fmt(fmt) || tokens < 0) return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        int64_t slot = slots[t];
        if (slot < 0 || slot >= num_pages * PAGE_TOKENS) continue;
        int64_t page = slot / PAGE_TOKENS, off = slot % PAGE_TOKENS;
        uint8_t *sec = cache + page * page_stride;
        float x[DIM], n[DIM];
        for (int i = 0; i < DIM; ++i) x[i] = bf16_to_f32(keys[t * k_row_stride + i]);
        orc_layernorm128(x, gamma, beta, eps, n);
        if (fmt == ORC_FMT_MXFP4) {
            mxfp4_of_128(n, sec + off * 64, sec + 64 * 64 + off * 4);
        } else if (fmt == ORC_FMT_FP8) {
            float s = fp8_of_128(n, sec + off * DIM);
            memcpy(sec + 64 * DIM + off * 4, &s, 4);
        } else {
            float s = fp8_of_128(n, sec + off * DIM);
            int ex;
            frexpf(s, &ex);  /* s = 0.5 * 2^ex exactly, so s = 2^(ex - 1) */
            uint8_t b = (uint8_t)(ex - 1 + 127);
            for (int i = 0; i < 4; ++i) sec[64 * DIM + off * 4 + i] = b;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* decode_layout ([fp4ops] decode_layout)                                   */
/* ------------------------------------------------------------------------ */

/* starts = [0, cumsum(query_lens)]. Row r belongs to the request that the
 * count of starts[1..R] <= r names (clamped to the last request); its key
 * bound is max(0, seq - qlen + r - start + 1). Under decode context
 * parallelism the bound is mapped into the rank-local key space of keys
 * interleaved across ranks in runs of `interleave`. Rows at or past the last
 * start are graph padding with bound 0. */
int orc_decode_layout(const int32_t *seq_lens, const int32_t *query_lens, int64_t num_requests,
                      int64_t num_rows, int dcp_rank, int dcp_world_size, int interleave,
                      int32_t *starts, int32_t *row_ends) {
    if (!(0 <= dcp_rank && dcp_rank < dcp_world_size) || interleave < 1 || num_rows < 0 ||
        num_requests < 0)
        return ORC_EINVAL;
    starts[0] = 0;
    for (int64_t i = 0; i < num_requests; ++i) starts[i + 1] = starts[i] + query_lens[i];
    for (int64_t row = 0; row < num_rows; ++row) {
        if (num_requests == 0) {
            row_ends[row] = 0;
            continue;
        }
        int64_t req = 0;
        while (req < num_requests && starts[req + 1] <= row) ++req;
        if (req > num_requests - 1) req = num_requests - 1;
        int64_t end = (int64_t)seq_lens[req] - query_lens[req] + row - starts[req] + 1;
        if (end < 0) end = 0;
        if (dcp_world_size > 1) {
            int64_t w = dcp_world_size, il = interleave;
            int64_t full = end / (w * il) * il;
            int64_t local = end - full * w - (int64_t)dcp_rank * il;
            if (local < 0) local = 0;
            if (local > il) local = il;
            end = full + local;
        }
        row_ends[row] = row < starts[num_requests] ? (int32_t)end : 0;
    }
    return ORC_OK;
}

/* Rows per verify tile ([fp4ops] decode_tile_size): one row of a tile costs
 * 4 B per key of FP32 logits, 24 B per selected key of selection scratch,
 * 64 B per head of quantized query and 256 B more; a tile gets as many rows
 * as fit in 32 rows of FP32 logits at max_model_len keys, and never fewer
 * than 32. Integer division rounds down. */
int64_t orc_decode_tile_size(int64_t max_model_len, int64_t width, int topk, int heads) {
    int64_t selected = topk < width ? (int64_t)topk : width;
    int64_t row_bytes = 4 * width + 24 * selected + 64 * (int64_t)heads + 256;
    if (row_bytes < 1) row_bytes = 1;
    int64_t budget = 32 * 4 * max_model_len;
    int64_t rows = budget / row_bytes;
    return rows < 32 ? 32 : rows;
}

/* ------------------------------------------------------------------------ */
/* score_paged ([fp4ops] score_paged; [idx] module text: MX scales stay     */
/* inside the logits contraction, head weights carry only the weight scale) */
/* ------------------------------------------------------------------------ */

static int nibble(const uint8_t *bytes, int col) {
    uint8_t b = bytes[col >> 1];
    return (col & 1) ? (b >> 4) : (b & 15);
}

/* One head's dot product q_h . k, exact: MXFP4 as integer block sums of
 * (2 E2M1) x (2 E2M1) scaled by 2^(eq + ek - 2); FP8 as the double sum of
 * exact E4M3 products times the key's scale (FP32, or 2^(byte - 127) from the
 * first of its four UE8M0 bytes for FP8_MX). */
static double head_dot(int fmt, const uint8_t *qrow, int heads, int h, const uint8_t *sec,
                       int64_t off) {
    if (fmt == ORC_FMT_MXFP4) {
        const uint8_t *qp = qrow + (int64_t)h * 64, *kp = sec + off * 64;
        const uint8_t *qs = qrow + (int64_t)heads * 64 + h * 4, *ks = sec + 64 * 64 + off * 4;
        double dot = 0.0;
        for (int g = 0; g < 4; ++g) {
            long acc = 0;
            for (int i = 0; i < 32; ++i) {
                int col = 32 * g + i;
                long a = (long)(2.0 * E2M1_TABLE[nibble(qp, col)]);
                long b = (long)(2.0 * E2M1_TABLE[nibble(kp, col)]);
                acc += a * b;
            }
            dot += ldexp((double)acc, ((int)qs[g] - 127) + ((int)ks[g] - 127) - 2);
        }
        return dot;
    } else {
        const uint8_t *qp = qrow + (int64_t)h * DIM, *kp = sec + off * DIM;
        double ks;
        if (fmt == ORC_FMT_FP8) {
            float f;
            memcpy(&f, sec + 64 * DIM + off * 4, 4);
            ks = (double)f;
        } else {
            ks = ldexp(1.0, (int)sec[64 * DIM + off * 4] - 127);
        }
        double dot = 0.0;
        for (int i = 0; i < DIM; ++i) dot += orc_e4m3_value(qp[i]) * orc_e4m3_value(kp[i]);
        return dot * ks;
    }
}

/* logit[r, p] = sum_h w[r, h] * max(0, q[r, h] . k[p]) for every row r of
 * request q and every key p < row_ends[r] (and < max_blocks * 64), key p read
 * from page block_table[q, p / 64] at offset p % 64. The head sum is carried
 * in double and rounded once to FP32. Keys on a page id outside
 * [0, num_pages) are skipped. If row_subset is not NULL only those rows are
 * scored. Other logits are left untouched. */
int orc_score_paged(int fmt, const uint8_t *q, int64_t q_row_stride, int heads,
                    const uint16_t *w, int64_t w_row_stride, const uint8_t *cache,
                    int64_t num_pages, int64_t page_stride, const int32_t *block_table,
                    int64_t num_requests, int64_t max_blocks, const int32_t *query_starts,
                    const int32_t *row_ends, int64_t num_rows, float *logits,
                    int64_t logits_row_stride, const int64_t *row_subset, int64_t n_subset) {
    if (!valid_fmt(fmt) || heads < 1) return ORC_EINVAL;
    if (!e4m3_ready) e4m3_fill();
    int64_t width = max_blocks * PAGE_TOKENS;
    for (int64_t req = 0; req < num_requests; ++req) {
        for (int64_t r = query_starts[req]; r < query_starts[req + 1] && r < num_rows; ++r) {
            if (row_subset) {
                int found = 0;
                for (int64_t i = 0; i < n_subset; ++i) found |= (row_subset[i] == r);
                if (!found) continue;
            }
            int64_t n = row_ends[r];
            if (n > width) n = width;
            const uint8_t *qrow = q + r * q_row_stride;
#pragma omp parallel for schedule(static)
            for (int64_t p = 0; p < n; ++p) {
                int64_t page = block_table[req * max_blocks + p / PAGE_TOKENS];
                if (page < 0 || page >= num_pages) continue;
                const uint8_t *sec = cache + page * page_stride;
                int64_t off = p % PAGE_TOKENS;
                double total = 0.0;
                for (int h = 0; h < heads; ++h) {
                    double dot = head_dot(fmt, qrow, heads, h, sec, off);
                    double relu = dot > 0.0 ? dot : 0.0;
                    total += (double)bf16_to_f32(w[r * w_row_stride + h]) * relu;
                }
                logits[r * logits_row_stride + p] = (float)total;
            }
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* topk (per-row selection after scoring; [ovl] module text: "scoring and   */
/* top-k"; ties go to the lower key index)                                  */
/* ------------------------------------------------------------------------ */

typedef struct {
    float v;
    int32_t i;
} scored_key;

/* Larger logit first; equal logits (-0 equals +0) by ascending key index. */
static int by_logit_then_index(const void *pa, const void *pb) {
    const scored_key *a = (const scored_key *)pa, *b = (const scored_key *)pb;
    if (a->v > b->v) return -1;
    if (a->v < b->v) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/* For each row: the key positions [0, min(row_ends[r], width)) sorted by
 * (logit descending, index ascending); the first min(k, n) go to indices[r],
 * in that order; the remaining entries of the k are -1. */
int orc_topk(const float *logits, int64_t rows, int64_t width, int64_t logits_row_stride,
             const int32_t *row_ends, int k, int32_t *indices, int64_t indices_row_stride) {
    if (rows < 0 || width < 0 || k < 1) return ORC_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t n = row_ends[r];
        if (n > width) n = width;
        if (n < 0) n = 0;
        scored_key *keys = (scored_key *)malloc((size_t)(n > 0 ? n : 1) * sizeof(scored_key));
        for (int64_t p = 0; p < n; ++p) {
            keys[p].v = logits[r * logits_row_stride + p];
            keys[p].i = (int32_t)p;
        }
        qsort(keys, (size_t)n, sizeof(scored_key), by_logit_then_index);
        for (int64_t j = 0; j < k; ++j)
            indices[r * indices_row_stride + j] = j < n ? keys[j].i : -1;
        free(keys);
    }
    return ORC_OK;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
