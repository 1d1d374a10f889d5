/*
 * CPU oracle for the NVFP4 W4A16 MTP draft-head hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library; the two meet only through the seeded input generators.
 *
 * Plain, slow and meant to be read next to the pages:
 *   [new.rs]      spark_model/layers/mtp_head/new.rs, `MtpHead::new`
 *   [mtp_head.rs] metrale_model_layers/layers/mtp_head.rs, `MtpHead::gemv`
 *   [v4_mtp.rs]   spark_model/layers/deepseek_v4_mtp.rs, `forward_one` and
 *                 `argmax_grammar_masked`
 *   [prefill.rs]  spark_model/layers/qwen3_attention/prefill_weights.rs,
 *                 `w4a16_gemm_m128_dispatch`
 * The pages name the steps (global absmax, block quantize, W4A16 GEMV, LM
 * head + argmax, top-k MoE, M=128 GEMM) but never spell out the NVFP4 bit
 * format; the format used here is the public one: E2M1 element codes, one
 * E4M3FN scale per 16 consecutive elements of a row, one fp32 global scale.
 *
 * Arithmetic: every fp32 operation is a single IEEE round-to-nearest-even
 * operation (compile with -ffp-contract=off); dot products accumulate in fp64,
 * where every term x * e2m1 * e4m3 is exact.
 *
 * Threads: the loops over independent outputs (rows of a GEMV, logits of
 * the LM head, rows of an expert's down projection, quantized rows) are
 * split over OpenMP threads; every output is computed by one thread in the
 * same order as with one thread, and every scan or sum across outputs (the
 * argmax, the log-sum-exp, the weighted expert sum) stays sequential, so
 * the results do not depend on the thread count.  orc_set_threads sets it.
 *
 * Parity status: every function below is pinned by tests (closed forms,
 * exhaustive codec sweeps, brute force with exact rationals, metamorphic
 * relations).  None is "parity unpinned".
 */
#include <math.h>
#include <float.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#include <omp.h>

#define ORC_API __attribute__((visibility("default")))

ORC_API void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
ORC_API int orc_get_threads(void) { return omp_get_max_threads(); }

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32 (a bf16 value is the upper half of an fp32 word, as the
 * CPU argmax in [v4_mtp.rs] `argmax_grammar_masked` decodes it).          */
/* ------------------------------------------------------------------ */
static float bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Round an fp32 value to bf16, nearest-even, by the definition: pick the
 * nearer of the two bf16 neighbours, ties to the even one. */
static uint16_t f32_to_bf16_rne(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lo = u & 0xFFFF0000u;          /* truncated neighbour (toward 0) */
    uint32_t rem = u & 0xFFFFu;
    uint16_t down = (uint16_t)(lo >> 16);
    if (rem < 0x8000u) return down;
    if (rem > 0x8000u) return (uint16_t)(down + 1);
    return (down & 1) ? (uint16_t)(down + 1) : down;
}

ORC_API float orc_bf16_round(float f) { return bf16_to_f32(f32_to_bf16_rne(f)); }

/* ------------------------------------------------------------------ */
/* Codecs (closed forms of the OCP FP4 E2M1 and FP8 E4M3FN formats).     */
/* ------------------------------------------------------------------ */

/* E2M1 code s e1 e0 m:  e == 0 -> 0.5*m ;  else 2^(e-1) * (1 + m/2). */
ORC_API double orc_e2m1_decode(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN byte s eeee mmm, bias 7: e == 0 -> m * 2^-9 ; else (1 + m/8) 2^(e-7);
 * 0x7F / 0xFF are NaN. */
ORC_API double orc_e4m3_decode(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Nearest E2M1 code to v: the magnitude is the nearest of the eight grid
 * points {0,.5,1,1.5,2,3,4,6}, ties to the even code, saturating at 6; the
 * sign bit is the sign of v (so -0 and small negatives give 0x8). */
ORC_API int orc_e2m1_encode(float v) {
    double a = fabs((double)v);
    int best = 0;
    if (a >= 6.0) {
        best = 7;
    } else {
        static double grid[8];
        static int grid_ready = 0;
        if (!grid_ready) {
            for (int c = 0; c < 8; ++c) grid[c] = orc_e2m1_decode(c);
            grid_ready = 1;
        }
        double bd = INFINITY;
        for (int c = 0; c < 8; ++c) {
            double d = fabs(a - grid[c]);
            if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
        }
    }
    return (signbit(v) ? 8 : 0) | best;
}

/* Nearest non-negative E4M3FN byte to s >= 0: round to nearest, ties to even
 * mantissa, subnormals kept (quantum 2^-9 below 2^-6), saturate to 448
 * (0x7E), never NaN.  Writes s = f * 2^E with f in [1,2) and rounds
 * s / 2^(E-3) to an integer, which is exact scaling by a power of two. */
ORC_API int orc_e4m3_encode(float s) {
    if (!(s > 0.0f)) return 0;
    if (s >= 448.0f) return 0x7E;
    int e;
    (void)frexp((double)s, &e);          /* s in [2^(e-1), 2^e) */
    int E = e - 1;
    if (E < -6) {                        /* subnormal range: multiples of 2^-9 */
        double q = rint(ldexp((double)s, 9));
        return (int)q;                   /* q == 8 is the smallest normal, 0x08 */
    }
    double q = rint(ldexp((double)s, 3 - E));   /* in [8, 16] */
    int code = ((E + 7) << 3) + ((int)q - 8);
    return code > 0x7E ? 0x7E : code;
}

/* Array forms of the two encoders (used by the exhaustive codec sweeps). */
ORC_API void orc_e2m1_encode_array(const float *v, int64_t count, uint8_t *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = (uint8_t)orc_e2m1_encode(v[i]);
}
ORC_API void orc_e4m3_encode_array(const float *s, int64_t count, uint8_t *out) {
    for (int64_t i = 0; i < count; ++i) out[i] = (uint8_t)orc_e4m3_encode(s[i]);
}

/* ------------------------------------------------------------------ */
/* NVFP4 quantizer: the two passes [new.rs] resolves as the kernels
 * `nvfp4_global_absmax` and `quantize_bf16_to_nvfp4` and runs for every
 * projection, router and expert matrix.                                  */
/* ------------------------------------------------------------------ */

/* Pass 1: global scales from the tensor's absolute maximum.
 * g_enc = 2688 / amax (6 * 448: the E2M1 maximum times the E4M3 maximum),
 * clamped to FLT_MAX, 0 when amax == 0;  g_dec = amax / 2688. */
ORC_API void orc_global_scales(const uint16_t *w, int64_t count, float out[3]) {
    float amax = 0.0f;
    for (int64_t i = 0; i < count; ++i) {
        float a = fabsf(bf16_to_f32(w[i]));
        if (a > amax) amax = a;
    }
    float g_enc = 0.0f;
    if (amax > 0.0f) {
        g_enc = 2688.0f / amax;
        if (g_enc > FLT_MAX) g_enc = FLT_MAX;
    }
    float g_dec = amax / 2688.0f;
    out[0] = g_dec;
    out[1] = g_enc;
    out[2] = amax;
}

/* Pass 2: per 16-element block of a row, an E4M3 scale; per element an E2M1
 * code, two per byte (even k in the low nibble), layout codes[n][k/2],
 * scales[n][k/16] (row-major, the packed [N, K/2] layout that
 * [prefill.rs] shows for NVFP4 weights).
 * glob_out = {g_dec, g_enc, amax}.  Requires k % 16 == 0. */
ORC_API void orc_quantize(const uint16_t *w, int64_t n, int64_t k,
                          uint8_t *codes, uint8_t *scales, float glob_out[3]) {
    float g[3];
    orc_global_scales(w, n * k, g);
    const float g_enc = g[1];
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t b = 0; b < k / 16; ++b) {
            const uint16_t *blk = w + r * k + b * 16;
            float bmax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(bf16_to_f32(blk[i]));
                if (a > bmax) bmax = a;
            }
            float t = bmax * g_enc;
            float s32 = t / 6.0f;
            int se = orc_e4m3_encode(s32);
            float sf = (float)orc_e4m3_decode(se);
            float inv = 0.0f;
            if (sf > 0.0f) {
                inv = g_enc / sf;
                if (inv > FLT_MAX) inv = FLT_MAX;
            }
            scales[r * (k / 16) + b] = (uint8_t)se;
            for (int i = 0; i < 16; i += 2) {
                float v0 = bf16_to_f32(blk[i]) * inv;
                float v1 = bf16_to_f32(blk[i + 1]) * inv;
                int c0 = orc_e2m1_encode(v0), c1 = orc_e2m1_encode(v1);
                codes[r * (k / 2) + b * 8 + i / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
    glob_out[0] = g[0];
    glob_out[1] = g[1];
    glob_out[2] = g[2];
}

/* Dequantized weight W^[n,k] = e2m1 * e4m3 * g_dec, in fp64 (the product
 * e2m1 * e4m3 has at most 6 significant bits). */
ORC_API void orc_dequantize(const uint8_t *codes, const uint8_t *scales, float g_dec,
                            int64_t n, int64_t k, double *out) {
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            uint8_t byte = codes[r * (k / 2) + c / 2];
            int code = (c & 1) ? (byte >> 4) : (byte & 15);
            out[r * k + c] = orc_e2m1_decode(code) *
                             orc_e4m3_decode(scales[r * (k / 16) + c / 16]) * (double)g_dec;
        }
}

/* ------------------------------------------------------------------ */
/* W4A16 GEMV / GEMM: y[m,n] = sum_k x[m,k] * W^[n,k], the `out = in @ W^T`
 * convention of [mtp_head.rs] `MtpHead::gemv` and of the prefill GEMM in
 * [prefill.rs].  fp64 sum of exact terms, one fp32 rounding at the end.   */
/* ------------------------------------------------------------------ */
/* Decode tables filled from the closed forms above (exact values; a lookup
 * instead of recomputing ldexp per element keeps the full-size cases fast). */
static double E2M1_TAB[16], E4M3_TAB[256];
static int tabs_ready = 0;
static void init_tabs(void) {
    if (tabs_ready) return;
    for (int c = 0; c < 16; ++c) E2M1_TAB[c] = orc_e2m1_decode(c);
    for (int b = 0; b < 256; ++b) E4M3_TAB[b] = orc_e4m3_decode(b);
    tabs_ready = 1;
}

/* sum_k x[k] * e2m1(code[k]) * e4m3(scale[k/16]) in fp64 (every term exact);
 * optionally also sum_k |term| for rounding-error bounds. */
static double dot_row2(const uint16_t *xrow, const uint8_t *crow, const uint8_t *srow, int64_t k,
                       double *abs_sum) {
    init_tabs();
    double acc = 0.0, aacc = 0.0;
    for (int64_t c = 0; c < k; ++c) {
        uint8_t byte = crow[c / 2];
        int code = (c & 1) ? (byte >> 4) : (byte & 15);
        double term = (double)bf16_to_f32(xrow[c]) * E2M1_TAB[code] * E4M3_TAB[srow[c / 16]];
        acc += term;
        aacc += fabs(term);
    }
    if (abs_sum) *abs_sum = aacc;
    return acc;
}

static double dot_row(const uint16_t *xrow, const uint8_t *crow, const uint8_t *srow, int64_t k) {
    return dot_row2(xrow, crow, srow, k, NULL);
}

ORC_API void orc_gemv(const uint16_t *x, int64_t m, const uint8_t *codes, const uint8_t *scales,
                      float g_dec, int64_t n, int64_t k, float *y) {
    init_tabs();
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t r = 0; r < n; ++r)
            y[i * n + r] = (float)((double)g_dec *
                                   dot_row(x + i * k, codes + r * (k / 2), scales + r * (k / 16), k));
}

/* Selected entries (mi[j], ni[j]) of the same product, for sizes where the
 * full product is too slow on a CPU. */
ORC_API void orc_gemm_sample(const uint16_t *x, const uint8_t *codes, const uint8_t *scales,
                             float g_dec, int64_t k, const int64_t *mi, const int64_t *ni,
                             int64_t count, float *out) {
    init_tabs();
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < count; ++j)
        out[j] = (float)((double)g_dec * dot_row(x + mi[j] * k, codes + ni[j] * (k / 2),
                                                 scales + ni[j] * (k / 16), k));
}

/* ------------------------------------------------------------------ */
/* LM head + argmax.  Rows [0, V) of the vocab weight are scored (the
 * reduced-vocab head of [new.rs] / [v4_mtp.rs]); the winner is found by the
 * ascending strict-greater scan of [v4_mtp.rs] `argmax_grammar_masked`:
 * start from best = -inf, index 0; a later equal value never replaces an
 * earlier one, NaN never wins, -0 == +0.  flags bit0 compares the logits
 * after rounding them to bf16 (the pages' GEMV -> bf16 logits -> argmax).
 * out_max is the fp32 logit of the winning row.                          */
/* ------------------------------------------------------------------ */
ORC_API void orc_lmhead_argmax(const uint16_t *h, int64_t m, const uint8_t *codes,
                               const uint8_t *scales, float g_dec, int64_t k, int64_t vrows,
                               uint32_t flags, int32_t *out_idx, float *out_max,
                               float *logits /* optional [m][vrows] */,
                               double *abs_bound /* optional [m][vrows]: g_dec * sum |terms| */) {
    init_tabs();
    float *lrow = (float *)malloc(sizeof(float) * (size_t)(vrows > 0 ? vrows : 1));
    for (int64_t i = 0; i < m; ++i) {
        float best = -INFINITY, bestlogit = 0.0f;
        int32_t bi = 0;
        int have = 0;
        /* the logits (independent), then the scan in ascending order */
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < vrows; ++r) {
            const uint8_t *crow = codes + r * (k / 2);
            const uint8_t *srow = scales + r * (k / 16);
            double asum = 0.0;
            lrow[r] = (float)((double)g_dec * dot_row2(h + i * k, crow, srow, k, &asum));
            if (logits) logits[i * vrows + r] = lrow[r];
            if (abs_bound) abs_bound[i * vrows + r] = (double)g_dec * asum;
        }
        for (int64_t r = 0; r < vrows; ++r) {
            const float logit = lrow[r];
            float key = (flags & 1u) ? orc_bf16_round(logit) : logit;
            if (key > best) { best = key; bi = (int32_t)r; bestlogit = logit; have = 1; }
        }
        if (!have && vrows > 0) {
            /* nothing beat -inf: index 0 and its logit */
            bestlogit = (float)((double)g_dec * dot_row(h + i * k, codes, scales, k));
        }
        out_idx[i] = bi;
        out_max[i] = bestlogit;
    }
    free(lrow);
}

/* ------------------------------------------------------------------ */
/* Top-1 log-probability of the LM head's argmax ([mtp_head.rs] `MtpHead`
 * fields: the batched argmax that also writes each row's top-1
 * log-probability, and the stored confidence of the last draft):
 *   lp = key[idx] - log(sum over r < vrows of exp(key[r]))
 * with key = the fp32 logit, or its bf16 rounding when flags bit 0 is set
 * (the same keys the argmax compares), idx the argmax of orc_lmhead_argmax.
 * The log-sum-exp is taken in fp64 after subtracting the largest key; any
 * NaN or infinite key makes lp NaN, as does a vocabulary of -inf keys.      */
/* ------------------------------------------------------------------ */
ORC_API void orc_lmhead_logprob(const uint16_t *h, int64_t m, const uint8_t *codes,
                                const uint8_t *scales, float g_dec, int64_t k, int64_t vrows,
                                uint32_t flags, double *out_lp) {
    init_tabs();
    float *key = (float *)malloc(sizeof(float) * (size_t)(vrows > 0 ? vrows : 1));
    for (int64_t i = 0; i < m; ++i) {
        float best = -INFINITY, kbest = 0.0f;
        int have = 0;
        double kmax = -INFINITY;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < vrows; ++r) {
            const uint8_t *crow = codes + r * (k / 2);
            const uint8_t *srow = scales + r * (k / 16);
            const float logit = (float)((double)g_dec * dot_row(h + i * k, crow, srow, k));
            key[r] = (flags & 1u) ? orc_bf16_round(logit) : logit;
        }
        for (int64_t r = 0; r < vrows; ++r) {
            if (key[r] > best) { best = key[r]; kbest = key[r]; have = 1; }
            if ((double)key[r] > kmax) kmax = (double)key[r];
        }
        if (!have && vrows > 0) kbest = key[0];   /* the argmax keeps index 0 */
        double sum = 0.0;
        for (int64_t r = 0; r < vrows; ++r) sum += exp((double)key[r] - kmax);
        out_lp[i] = (double)kbest - (kmax + log(sum));
    }
    free(key);
}

/* ------------------------------------------------------------------ */
/* Grammar-masked LM-head argmax ([v4_mtp.rs] `argmax_grammar_masked`):
 * token r is allowed when bit r % 32 of mask word r / 32 of the row's mask
 * is set (mask_words words per activation row); the ascending strict-greater
 * scan runs over the allowed tokens only and starts at index 0 with -inf, so
 * an empty allowed set (or one whose keys are all -inf or NaN) gives index 0.
 * out_max is the fp32 logit of the returned row.  out_lp (optional) is the
 * top-1 log-probability over the allowed tokens: key[idx] minus the
 * log-sum-exp of the allowed keys, NaN when that set has no finite mass.
 * mask == NULL allows every row (then this equals orc_lmhead_argmax and
 * orc_lmhead_logprob).                                                  */
/* ------------------------------------------------------------------ */
ORC_API void orc_lmhead_masked(const uint16_t *h, int64_t m, const uint8_t *codes,
                               const uint8_t *scales, float g_dec, int64_t k, int64_t vrows,
                               uint32_t flags, const uint32_t *mask, int64_t mask_words,
                               int32_t *out_idx, float *out_max, double *out_lp) {
    float *key = (float *)malloc(sizeof(float) * (size_t)(vrows > 0 ? vrows : 1));
    float *logit = (float *)malloc(sizeof(float) * (size_t)(vrows > 0 ? vrows : 1));
    char *allowed = (char *)malloc((size_t)(vrows > 0 ? vrows : 1));
    init_tabs();
    for (int64_t i = 0; i < m; ++i) {
        float best = -INFINITY;
        int32_t bi = 0;
        double kmax = -INFINITY;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < vrows; ++r) {
            const uint8_t *crow = codes + r * (k / 2);
            const uint8_t *srow = scales + r * (k / 16);
            logit[r] = (float)((double)g_dec * dot_row(h + i * k, crow, srow, k));
            key[r] = (flags & 1u) ? orc_bf16_round(logit[r]) : logit[r];
            allowed[r] = mask == NULL ||
                         (r / 32 < mask_words && ((mask[i * mask_words + r / 32] >> (r % 32)) & 1u));
        }
        for (int64_t r = 0; r < vrows; ++r) {
            if (!allowed[r]) continue;
            if (key[r] > best) { best = key[r]; bi = (int32_t)r; }
            if ((double)key[r] > kmax) kmax = (double)key[r];
        }
        out_idx[i] = bi;
        out_max[i] = vrows > 0 ? logit[bi] : 0.0f;
        if (out_lp) {
            double sum = 0.0;
            for (int64_t r = 0; r < vrows; ++r)
                if (allowed[r]) sum += exp((double)key[r] - kmax);
            /* an empty allowed set has no probability mass: not measured */
            out_lp[i] = sum > 0.0 ? (double)key[bi] - (kmax + log(sum)) : NAN;
        }
    }
    free(key);
    free(logit);
    free(allowed);
}

/* Embedding rows of the draft tokens ([mtp_head.rs] `embed_from_argmax`,
 * which also stores the draft id on the device for deferred readback):
 * out[i][:] = table[idx[i]][:] (bf16 rows of `hidden`), a zero row for an
 * index outside [0, vocab).                                               */
ORC_API void orc_embed_rows(const int32_t *idx, int64_t m, const uint16_t *table, int64_t vocab,
                            int64_t hidden, uint16_t *out) {
    for (int64_t i = 0; i < m; ++i)
        for (int64_t c = 0; c < hidden; ++c)
            out[i * hidden + c] = (idx[i] >= 0 && idx[i] < vocab) ? table[(int64_t)idx[i] * hidden + c] : 0;
}

/* ------------------------------------------------------------------ */
/* MoE FFN of the draft head: top-k experts by router logit, softmax over
 * the selected logits, SiLU-gated expert MLP, weighted sum
 * ([new.rs]: `moe_topk_softmax`, `moe_silu_mul`, `moe_weighted_sum_blend`,
 * NVFP4 expert gate/up [inter, h] and down [h, inter]).
 * Expert e's matrices sit at gate_codes + e*I*H/2 etc.; g_dec per expert.  */
/* ------------------------------------------------------------------ */
ORC_API void orc_moe(const uint16_t *x, int64_t m, const float *router, int64_t E, int64_t topk,
                     int64_t H, int64_t I,
                     const uint8_t *gc, const uint8_t *gs, const float *gdec,
                     const uint8_t *uc, const uint8_t *us, const float *udec,
                     const uint8_t *dc, const uint8_t *ds, const float *ddec,
                     float *y, int32_t *ids, float *wts) {
    init_tabs();
    float *g = (float *)malloc(sizeof(float) * I);
    float *u = (float *)malloc(sizeof(float) * I);
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * I);
    double *acc = (double *)malloc(sizeof(double) * H);
    char *taken = (char *)malloc(E);
    for (int64_t t = 0; t < m; ++t) {
        const float *lg = router + t * E;
        /* top-k: repeatedly take the largest remaining logit, lowest id on ties */
        memset(taken, 0, E);
        for (int64_t j = 0; j < topk; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || lg[e] > lg[best]) best = e;
            }
            taken[best] = 1;
            ids[t * topk + j] = (int32_t)best;
        }
        /* softmax over the selected logits */
        double lmax = lg[ids[t * topk]];
        double den = 0.0;
        for (int64_t j = 0; j < topk; ++j) den += exp((double)lg[ids[t * topk + j]] - lmax);
        for (int64_t j = 0; j < topk; ++j)
            wts[t * topk + j] = (float)(exp((double)lg[ids[t * topk + j]] - lmax) / den);
        for (int64_t h = 0; h < H; ++h) acc[h] = 0.0;
        for (int64_t j = 0; j < topk; ++j) {
            int64_t e = ids[t * topk + j];
            orc_gemv(x + t * H, 1, gc + e * I * (H / 2), gs + e * I * (H / 16), gdec[e], I, H, g);
            orc_gemv(x + t * H, 1, uc + e * I * (H / 2), us + e * I * (H / 16), udec[e], I, H, u);
            for (int64_t i = 0; i < I; ++i) {
                double gi = g[i];
                double act = gi / (1.0 + exp(-gi)) * (double)u[i];
                a[i] = f32_to_bf16_rne((float)act);
            }
#pragma omp parallel for schedule(static)
            for (int64_t h = 0; h < H; ++h) {
                float d = (float)((double)ddec[e] *
                                  dot_row(a, dc + e * H * (I / 2) + h * (I / 2),
                                          ds + e * H * (I / 16) + h * (I / 16), I));
                acc[h] += (double)wts[t * topk + j] * (double)d;   /* slot order j per h */
            }
        }
        for (int64_t h = 0; h < H; ++h) y[t * H + h] = (float)acc[h];
    }
    free(g); free(u); free(a); free(acc); free(taken);
}

/* ------------------------------------------------------------------ */
/* The complete MoE layer of the draft head ([new.rs] `MtpHead::new`: the
 * router `moe_gate` quantized to NVFP4 next to the routed experts, a shared
 * expert (gate/up/down, NVFP4) and its `shared_expert_gate`, combined by
 * `moe_weighted_sum_blend`):
 *   logits = router x (fp32, the NVFP4 GEMV of orc_gemv);
 *   y      = routed MoE of orc_moe on those logits
 *            + sigmoid(sgate . x) * shared(x),
 *   shared(x) = down_s(bf16(silu(gate_s x) * up_s x)),
 * with sgate a bf16 vector of H (the gate weight kept in bf16); sgate NULL
 * means an ungated shared expert (factor 1).  The routed part is rounded
 * to fp32 by orc_moe before the shared term is added in fp64.            */
/* ------------------------------------------------------------------ */
ORC_API void orc_moe_layer(const uint16_t *x, int64_t m, const uint8_t *rc, const uint8_t *rs, float rdec,
                           int64_t E, int64_t topk, int64_t H, int64_t I,
                           const uint8_t *gc, const uint8_t *gs, const float *gdec,
                           const uint8_t *uc, const uint8_t *us, const float *udec,
                           const uint8_t *dc, const uint8_t *ds, const float *ddec,
                           const uint8_t *sgc, const uint8_t *sgs, float sgdec,
                           const uint8_t *suc, const uint8_t *sus, float sudec,
                           const uint8_t *sdc, const uint8_t *sds, float sddec, int64_t Is,
                           const uint16_t *sgate, float *y, int32_t *ids, float *wts, float *logits) {
    orc_gemv(x, m, rc, rs, rdec, E, H, logits);
    orc_moe(x, m, logits, E, topk, H, I, gc, gs, gdec, uc, us, udec, dc, ds, ddec, y, ids, wts);
    float *g = (float *)malloc(sizeof(float) * Is);
    float *u = (float *)malloc(sizeof(float) * Is);
    uint16_t *a = (uint16_t *)malloc(sizeof(uint16_t) * Is);
    for (int64_t t = 0; t < m; ++t) {
        const uint16_t *xt = x + t * H;
        double sg = 1.0;
        if (sgate) {
            double z = 0.0;
            for (int64_t h = 0; h < H; ++h) z += (double)bf16_to_f32(sgate[h]) * (double)bf16_to_f32(xt[h]);
            sg = 1.0 / (1.0 + exp(-z));
        }
        orc_gemv(xt, 1, sgc, sgs, sgdec, Is, H, g);
        orc_gemv(xt, 1, suc, sus, sudec, Is, H, u);
        for (int64_t i = 0; i < Is; ++i) {
            double gi = g[i];
            a[i] = f32_to_bf16_rne((float)(gi / (1.0 + exp(-gi)) * (double)u[i]));
        }
#pragma omp parallel for schedule(static)
        for (int64_t h = 0; h < H; ++h) {
            float d = (float)((double)sddec * dot_row(a, sdc + h * (Is / 2), sds + h * (Is / 16), Is));
            y[t * H + h] = (float)((double)y[t * H + h] + sg * (double)d);
        }
    }
    free(g); free(u); free(a);
}
