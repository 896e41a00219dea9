/*
 * oracle.c -- plain, slow FP64 CPU reference for E4M3 paged speculative-verify
 * attention with split partials.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path links, loads or calls
 * this file. It is used by tests/, by __graft_entry__.smoke() and by the
 * cpu_baseline leg of bench.py. It shares no code, header, table or constant
 * with the HIP library under paged_fp8_split_amd/.
 *
 * What it computes follows the pages' statement of the method:
 *  - "[Kernel][SM70] Add opt-in E4M3 grouped attention with FP32 partials",
 *    final-status section (revision 3 bullet): every KV partition keeps its
 *    running max, its sum and its *unnormalized* PV product until one final
 *    combine, which rescales the partials and normalizes once.
 *  - "[Kernel] Finalize the audited TP2 DFlash2 31/29 ms endpoint", Purpose:
 *    keys are consumed in 64-key partitions in a fixed (ascending) order;
 *    Test Result: an exact E4M3 decoder checked over all byte values and an
 *    FP64 reference.
 *  - "[Bugfix] Use FP32 state and E4M3 defaults for DFlash2", Purpose: KV is
 *    stored as FP8 E4M3, the query and the final activations are FP16.
 *
 * Readings where the pages are silent (each is listed in the design doc):
 *  - E4M3 is the OCP "FN" variant: bias 7, no infinities, S.1111.111 = NaN,
 *    largest finite 448.
 *  - A request's live length L includes its q draft tokens; draft row i
 *    (0-based) sees the first n_i = L - q + i + 1 tokens (clamped to [0, L]).
 *    A row that sees no token outputs +0.0.
 *  - Partitions are absolute token ranges [p*T, (p+1)*T) of the row.
 *  - Scales multiply the decoded bytes exactly (no re-rounding).
 *
 * Everything here is FP64 with plain loops in the order the method states:
 * decode, score, per-partition (max, sum, unnormalized PV), then combine.
 * Built with -O2 and without -ffast-math (the build script fixes the flags).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-2)

/* OCP E4M3FN byte -> exact value. s = sign bit, e = 4-bit biased exponent,
 * m = 3-bit mantissa. e == 0 is subnormal: m/8 * 2^(1-7). e == 15 with m == 7
 * is NaN; every other code is normal: (1 + m/8) * 2^(e-7). */
double oracle_e4m3_value(uint32_t byte) {
    const int s = (int)((byte >> 7) & 1u);
    const int e = (int)((byte >> 3) & 15u);
    const int m = (int)(byte & 7u);
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - 7);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* IEEE binary16 bit pattern -> exact value. */
double oracle_fp16_value(uint32_t bits) {
    const int s = (int)((bits >> 15) & 1u);
    const int e = (int)((bits >> 10) & 31u);
    const int m = (int)(bits & 1023u);
    double mag;
    if (e == 31) {
        if (m) return NAN;
        return s ? -INFINITY : INFINITY;
    }
    if (e == 0)
        mag = ldexp((double)m, -24);
    else
        mag = ldexp(1024.0 + (double)m, e - 25);
    return s ? -mag : mag;
}

/* Fill out[0..255] with the decoded value of every byte. */
void oracle_e4m3_table(double* out) {
    for (uint32_t b = 0; b < 256; ++b) out[b] = oracle_e4m3_value(b);
}

/* E5M2 byte -> exact value: the IEEE-style 8-bit format with a 5-bit
 * exponent (bias 15) and a 2-bit mantissa, kept beside E4M3 as an explicit
 * alternative KV format ("[Bugfix] Use FP32 state and E4M3 defaults for
 * DFlash2", Purpose: E4M3 is the default, E5M2 stays available on request;
 * "[Kernel][SM70] Add opt-in E4M3 grouped attention with FP32 partials",
 * historical scope: explicit E5M2 routes are kept). e == 0 is subnormal:
 * m/4 * 2^(1-15); e == 31 is infinity (m == 0) or NaN; otherwise
 * (1 + m/4) * 2^(e-15). Largest finite value 57344. */
double oracle_e5m2_value(uint32_t byte) {
    const int s = (int)((byte >> 7) & 1u);
    const int e = (int)((byte >> 2) & 31u);
    const int m = (int)(byte & 3u);
    double mag;
    if (e == 31) {
        if (m) return NAN;
        return s ? -INFINITY : INFINITY;
    }
    if (e == 0)
        mag = ldexp((double)m / 4.0, 1 - 15);
    else
        mag = ldexp(1.0 + (double)m / 4.0, e - 15);
    return s ? -mag : mag;
}

#define ORACLE_KV_E4M3 0
#define ORACLE_KV_E5M2 1

/* Decoded value of every byte of KV format `format`; 0 on success. */
int oracle_kv_table(int32_t format, double* out) {
    if (format != ORACLE_KV_E4M3 && format != ORACLE_KV_E5M2) return ORACLE_ERR_ARG;
    for (uint32_t b = 0; b < 256; ++b)
        out[b] = format == ORACLE_KV_E5M2 ? oracle_e5m2_value(b) : oracle_e4m3_value(b);
    return ORACLE_OK;
}

/* Number of keys draft row i of a request with live length L may attend to. */
int64_t oracle_visible_keys(int64_t live_len, int32_t q, int32_t row) {
    int64_t n = live_len - (int64_t)q + (int64_t)row + 1;
    if (n < 0) n = 0;
    if (n > live_len) n = live_len;
    return n;
}

/*
 * The verify attention.
 *
 * Shapes (all host memory):
 *   q_fp16      [batch, q, num_q_heads, head_dim]  IEEE half bit patterns
 *   k_pool/v_pool  byte pools addressed as
 *                  page*page_stride + slot*token_stride + kv_head*head_stride + d
 *   k_scale/v_scale [num_kv_heads] FP32
 *   block_table [batch, max_pages_per_row] physical page of each logical page
 *   live_len    [batch]
 *   head_map    [num_q_heads] query head -> KV head
 *   unit_mask   [batch * num_q_heads] or NULL: compute only units whose mask
 *               byte is non-zero (others are left untouched)
 *   out         [batch, q, num_q_heads, head_dim] FP64 (unrounded result)
 *
 * kv_format selects how the pool bytes decode: 0 = E4M3FN (the default
 * format of the method), 1 = E5M2.
 *
 * partition_tokens <= 0 means a single partition per row (the unsplit
 * softmax). Returns ORACLE_OK or a negative error code.
 */
int oracle_verify(int32_t batch, int32_t q, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t page_size, int32_t max_pages_per_row,
                  int32_t num_pool_pages, int32_t partition_tokens, int64_t page_stride,
                  int64_t token_stride, int64_t head_stride, const uint16_t* q_fp16,
                  const uint8_t* k_pool, const uint8_t* v_pool, const float* k_scale,
                  const float* v_scale, const int32_t* block_table, const int32_t* live_len,
                  const int32_t* head_map, const uint8_t* unit_mask, double sm_scale,
                  double* out, int32_t num_threads, int32_t kv_format) {
    if (batch < 0 || q < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
        page_size < 1 || max_pages_per_row < 0 || num_pool_pages < 0)
        return ORACLE_ERR_ARG;
    if (!q_fp16 || !k_pool || !v_pool || !k_scale || !v_scale || !block_table || !live_len ||
        !head_map || !out)
        return ORACLE_ERR_ARG;
    for (int32_t h = 0; h < num_q_heads; ++h)
        if (head_map[h] < 0 || head_map[h] >= num_kv_heads) return ORACLE_ERR_ARG;

    double table[256];
    if (oracle_kv_table(kv_format, table) != ORACLE_OK) return ORACLE_ERR_ARG;

    const int64_t capacity = (int64_t)max_pages_per_row * page_size;
    const int64_t units = (int64_t)batch * num_q_heads;
    int status = ORACLE_OK;

#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#else
    (void)num_threads;
#endif

#pragma omp parallel
    {
        double* qrow = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* khat = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* vhat = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
        double* part_m = NULL;
        double* part_l = NULL;
        double* part_a = NULL;
        double* sbuf = NULL;
        int64_t part_cap = 0;
        int64_t sbuf_cap = 0;
        int local_err = (!qrow || !khat || !vhat || !acc);
        int bad_page = 0;

#pragma omp for schedule(dynamic, 1)
        for (int64_t unit = 0; unit < units * q; ++unit) {
            if (local_err || bad_page) continue;
            const int64_t bh = unit / q;
            const int32_t row = (int32_t)(unit % q);
            const int32_t b = (int32_t)(bh / num_q_heads);
            const int32_t h = (int32_t)(bh % num_q_heads);
            if (unit_mask && !unit_mask[bh]) continue;
            const int32_t g = head_map[h];
            double* dst = out + (((int64_t)b * q + row) * num_q_heads + h) * head_dim;

            int64_t L = live_len[b];
            if (L < 0) L = 0;
            if (L > capacity) L = capacity;
            const int64_t n = oracle_visible_keys(L, q, row);
            if (n == 0) {
                for (int32_t d = 0; d < head_dim; ++d) dst[d] = 0.0;
                continue;
            }

            /* The draft query row, FP16 -> FP64 exactly. */
            const uint16_t* qsrc = q_fp16 + (((int64_t)b * q + row) * num_q_heads + h) * head_dim;
            for (int32_t d = 0; d < head_dim; ++d) qrow[d] = oracle_fp16_value(qsrc[d]);

            const int64_t T = partition_tokens > 0 ? partition_tokens : n;
            const int64_t nparts = (n + T - 1) / T;
            if (nparts > part_cap) {
                free(part_m);
                free(part_l);
                free(part_a);
                part_m = (double*)malloc(sizeof(double) * (size_t)nparts);
                part_l = (double*)malloc(sizeof(double) * (size_t)nparts);
                part_a = (double*)malloc(sizeof(double) * (size_t)nparts * (size_t)head_dim);
                part_cap = nparts;
                if (!part_m || !part_l || !part_a) {
                    local_err = 1;
                    part_cap = 0;
                    continue;
                }
            }

            if (T > sbuf_cap) {
                free(sbuf);
                sbuf = (double*)malloc(sizeof(double) * (size_t)T);
                sbuf_cap = T;
                if (!sbuf) {
                    local_err = 1;
                    sbuf_cap = 0;
                    continue;
                }
            }

            /* Per partition, ascending: max score, sum of exp, unnormalized PV. */
            for (int64_t p = 0; p < nparts; ++p) {
                const int64_t j0 = p * T;
                const int64_t j1 = (j0 + T < n) ? j0 + T : n;
                double* a = part_a + p * head_dim;
                /* scores of the partition's keys and their max */
                double m = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    const int32_t page = block_table[(int64_t)b * max_pages_per_row + j / page_size];
                    if (page < 0 || page >= num_pool_pages) {
                        bad_page = 1;
                        break;
                    }
                    const int64_t base = (int64_t)page * page_stride + (j % page_size) * token_stride +
                                         (int64_t)g * head_stride;
                    double s = 0.0;
                    for (int32_t d = 0; d < head_dim; ++d) {
                        khat[d] = table[k_pool[base + d]] * (double)k_scale[g];
                        s += qrow[d] * khat[d];
                    }
                    s *= sm_scale;
                    sbuf[j - j0] = s;
                    if (s > m) m = s;
                }
                if (bad_page) break;
                /* weights relative to that max: their sum and the unnormalized PV */
                double l = 0.0;
                for (int32_t d = 0; d < head_dim; ++d) a[d] = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    const int32_t page = block_table[(int64_t)b * max_pages_per_row + j / page_size];
                    const int64_t base = (int64_t)page * page_stride + (j % page_size) * token_stride +
                                         (int64_t)g * head_stride;
                    const double w = exp(sbuf[j - j0] - m);
                    l += w;
                    for (int32_t d = 0; d < head_dim; ++d) {
                        vhat[d] = table[v_pool[base + d]] * (double)v_scale[g];
                        a[d] += w * vhat[d];
                    }
                }
                part_m[p] = m;
                part_l[p] = l;
            }

            if (bad_page) continue;

            /* Final combine: rescale each partition to the global max, sum in
             * partition order, normalize once. */
            double M = -INFINITY;
            for (int64_t p = 0; p < nparts; ++p)
                if (part_m[p] > M) M = part_m[p];
            double l = 0.0;
            for (int32_t d = 0; d < head_dim; ++d) acc[d] = 0.0;
            for (int64_t p = 0; p < nparts; ++p) {
                const double f = exp(part_m[p] - M);
                l += f * part_l[p];
                const double* a = part_a + p * head_dim;
                for (int32_t d = 0; d < head_dim; ++d) acc[d] += f * a[d];
            }
            for (int32_t d = 0; d < head_dim; ++d) dst[d] = acc[d] / l;
        }

        if (local_err) {
#pragma omp atomic write
            status = ORACLE_ERR_NOMEM;
        }
        if (bad_page) {
#pragma omp atomic write
            status = ORACLE_ERR_ARG;
        }
        free(qrow);
        free(khat);
        free(vhat);
        free(acc);
        free(part_m);
        free(part_l);
        free(part_a);
        free(sbuf);
    }
    return status;
}

/* Threads an OpenMP parallel region would use (for reporting). */
int32_t oracle_max_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Quantize-on-write: the K/V of a request's q draft tokens, FP16, stored into
 * its paged E4M3 pool with the per-KV-head scale (the step before verify;
 * "[Kernel] Preserve DFlash2 sampling precision ...", Purpose: deferred
 * accepted-slot writes; "[Bugfix] Use FP32 state ...", Test Plan: KV scaling).
 *
 * Readings (listed in the design doc): the stored byte is the E4M3FN code nearest
 * to the FP32 quotient x / scale (IEEE single division, correctly rounded),
 * ties to the even code, saturating at +-448 (infinities too); a NaN quotient
 * stores 0x7F. Draft row i of request b lands at token L_b - q + i; rows that
 * would land before token 0 (L_b < q) are not written.
 */

/* E4M3FN code nearest to the FP32 value v, ties to even, saturating. */
uint32_t oracle_e4m3_encode(float v) {
    if (isnan(v)) return 0x7Fu;
    const uint32_t sign = signbit(v) ? 0x80u : 0u;
    const double a = fabs((double)v);
    if (a >= 448.0) return sign | 0x7Eu;  /* 448 = S.1111.110 */
    if (a < ldexp(1.0, -6)) {
        /* subnormal grid: multiples of 2^-9; rounding to 8 gives the smallest normal */
        const double n = nearbyint(a * 512.0);
        return sign | (uint32_t)n;
    }
    int e = (int)floor(log2(a));
    /* guard against log2 rounding at exact powers of two */
    if (ldexp(1.0, e) > a) e -= 1;
    if (ldexp(1.0, e + 1) <= a) e += 1;
    double sig = nearbyint(a / ldexp(1.0, e - 3)); /* 8 .. 16 */
    if (sig >= 16.0) {
        sig = 8.0;
        e += 1;
    }
    if (e > 8 || (e == 8 && sig > 14.0)) return sign | 0x7Eu;
    return sign | (uint32_t)(((e + 7) << 3) | ((int)sig - 8));
}

/* E5M2 code nearest to the FP32 value v, ties to even, saturating at
 * +-57344 (infinities too); NaN -> 0x7F (a NaN code of E5M2 as well). The
 * same reading as the E4M3 encoder, on E5M2's grid: normals (1 + m/4) *
 * 2^e for e in [-14, 15], subnormals multiples of 2^-16. */
uint32_t oracle_e5m2_encode(float v) {
    if (isnan(v)) return 0x7Fu;
    const uint32_t sign = signbit(v) ? 0x80u : 0u;
    const double a = fabs((double)v);
    if (a >= 57344.0) return sign | 0x7Bu; /* 57344 = S.11110.11 */
    if (a < ldexp(1.0, -14)) {
        /* subnormal grid: multiples of 2^-16; rounding to 4 gives the smallest normal */
        const double n = nearbyint(a * 65536.0);
        return sign | (uint32_t)n;
    }
    int e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) e -= 1;
    if (ldexp(1.0, e + 1) <= a) e += 1;
    double sig = nearbyint(a / ldexp(1.0, e - 2)); /* 4 .. 8 */
    if (sig >= 8.0) {
        sig = 4.0;
        e += 1;
    }
    if (e > 15 || (e == 15 && sig > 7.0)) return sign | 0x7Bu;
    return sign | (uint32_t)(((e + 15) << 2) | ((int)sig - 4));
}

/* FP16 bits x stored with scale s in KV format `format`: the code of (float)x / s. */
uint32_t oracle_quantize_fp16(uint32_t bits, float scale, int32_t format) {
    const float x = (float)oracle_fp16_value(bits);
    const float quotient = x / scale;
    return format == ORACLE_KV_E5M2 ? oracle_e5m2_encode(quotient) : oracle_e4m3_encode(quotient);
}

/*
 * Write the draft tokens' K and V into the pools (in place).
 *   k_new/v_new [batch, q, num_kv_heads, head_dim] IEEE half bit patterns
 *   pools, strides, block_table, live_len as for oracle_verify; lengths are
 *   clamped into [0, max_pages_per_row * page_size].
 *   kv_format 0 stores E4M3FN codes, 1 stores E5M2 codes.
 * Returns ORACLE_OK, or ORACLE_ERR_ARG for a block-table entry outside the
 * pool or an unknown format.
 */
int oracle_kv_append(int32_t batch, int32_t q, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                     int32_t max_pages_per_row, int32_t num_pool_pages, int64_t page_stride,
                     int64_t token_stride, int64_t head_stride, const uint16_t* k_new, const uint16_t* v_new,
                     const float* k_scale, const float* v_scale, const int32_t* block_table,
                     const int32_t* live_len, uint8_t* k_pool, uint8_t* v_pool, int32_t kv_format) {
    if (kv_format != ORACLE_KV_E4M3 && kv_format != ORACLE_KV_E5M2) return ORACLE_ERR_ARG;
    const int64_t capacity = (int64_t)max_pages_per_row * page_size;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = live_len[b];
        if (L < 0) L = 0;
        if (L > capacity) L = capacity;
        for (int32_t i = 0; i < q; ++i) {
            const int64_t t = L - q + i;
            if (t < 0) continue;
            const int32_t page = block_table[(int64_t)b * max_pages_per_row + t / page_size];
            if (page < 0 || page >= num_pool_pages) return ORACLE_ERR_ARG;
            const int64_t base = (int64_t)page * page_stride + (t % page_size) * token_stride;
            for (int32_t g = 0; g < num_kv_heads; ++g) {
                const int64_t src = (((int64_t)b * q + i) * num_kv_heads + g) * head_dim;
                for (int32_t d = 0; d < head_dim; ++d) {
                    const int64_t dst = base + (int64_t)g * head_stride + d;
                    k_pool[dst] = (uint8_t)oracle_quantize_fp16(k_new[src + d], k_scale[g], kv_format);
                    v_pool[dst] = (uint8_t)oracle_quantize_fp16(v_new[src + d], v_scale[g], kv_format);
                }
            }
        }
    }
    return ORACLE_OK;
}

/* IEEE binary16 bits of the double v rounded to nearest, ties to even
 * (overflow to infinity, gradual underflow, NaN -> 0x7E00). */
uint32_t oracle_fp16_rne(double v) {
    if (isnan(v)) return 0x7E00u;
    const uint32_t sign = signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (a >= 65520.0) return sign | 0x7C00u; /* halfway to 2^16 and above: infinity */
    if (a < ldexp(1.0, -14)) {
        const double n = nearbyint(a * 16777216.0); /* multiples of 2^-24; 1024 is the smallest normal */
        return sign | (uint32_t)n;
    }
    int e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) e -= 1;
    if (ldexp(1.0, e + 1) <= a) e += 1;
    double sig = nearbyint(a / ldexp(1.0, e - 10)); /* 1024 .. 2048 */
    if (sig >= 2048.0) {
        sig = 1024.0;
        e += 1;
    }
    if (e > 15) return sign | 0x7C00u;
    return sign | (uint32_t)(((e + 15) << 10) | ((int)sig - 1024));
}

/*
 * Paged E4M3 -> FP16 bridge ("[Kernel][SM70] Add opt-in E4M3 grouped
 * attention with FP32 partials", Scope list: a standalone call that turns
 * the paged FP8 cache into FP16): out[b][t][g][d] = FP16 bits of dec(byte) * scale[g] rounded once to
 * nearest even for t < live_len[b], +0.0 beyond, with dec the decoder of
 * kv_format (0 = E4M3FN, 1 = E5M2). scale == NULL means 1.
 * out is [batch, max_pages_per_row * page_size, num_kv_heads, head_dim].
 */
int oracle_dequant(int32_t batch, int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                   int32_t max_pages_per_row, int32_t num_pool_pages, int64_t page_stride, int64_t token_stride,
                   int64_t head_stride, const uint8_t* pool, const float* scale, const int32_t* block_table,
                   const int32_t* live_len, uint16_t* out, int32_t kv_format) {
    double table[256];
    if (oracle_kv_table(kv_format, table) != ORACLE_OK) return ORACLE_ERR_ARG;
    const int64_t capacity = (int64_t)max_pages_per_row * page_size;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t L = live_len[b];
        if (L < 0) L = 0;
        if (L > capacity) L = capacity;
        for (int64_t t = 0; t < capacity; ++t) {
            for (int32_t g = 0; g < num_kv_heads; ++g) {
                uint16_t* dst = out + ((b * capacity + t) * num_kv_heads + g) * head_dim;
                if (t >= L) {
                    for (int32_t d = 0; d < head_dim; ++d) dst[d] = 0;
                    continue;
                }
                const int32_t page = block_table[(int64_t)b * max_pages_per_row + t / page_size];
                if (page < 0 || page >= num_pool_pages) return ORACLE_ERR_ARG;
                const uint8_t* src = pool + (int64_t)page * page_stride + (t % page_size) * token_stride +
                                     (int64_t)g * head_stride;
                const double s = scale ? (double)scale[g] : 1.0;
                for (int32_t d = 0; d < head_dim; ++d)
                    dst[d] = (uint16_t)oracle_fp16_rne(table[src[d]] * s);
            }
        }
    }
    return ORACLE_OK;
}
