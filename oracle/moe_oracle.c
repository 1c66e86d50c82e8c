/*
 * moe_oracle.c -- CPU oracle for one MoE layer (dispatch -> L1 -> SwiGLU*w ->
 * FP8 requant -> L2 -> combine).  TEST INFRASTRUCTURE ONLY: tests, the smoke
 * check and the benchmark's CPU-baseline leg load it; the HIP library never
 * does.  Plain C11, OpenMP for the outer loops only, no blocking, no fusion.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -shared -fPIC
 * (-ffp-contract=off keeps every multiply and add separately rounded, as the
 * step definitions below state them).
 *
 * Page tags [P1]/[P2]/[P3] are defined in moe_oracle.h.
 *
 * Readings taken where the pages are silent (each is also listed with the
 * design notes of the repository):
 *  - UE8M0 scale choice: the pages only say an absolute maximum is reduced
 *    before the FP8 cast ([P1], "complete compute pipeline" snippet, steps 3
 *    and 4).  Reading: the scale is the smallest power of two 2^(b-127) with
 *    amax <= 448 * 2^(b-127), so no value saturates; amax = 0 gives b = 0.
 *  - Groups of 32 along K for every scale (recipe (1,1,32), [P2] section 2).
 *  - GEMM outputs are the exact dot product of the dequantised operands,
 *    rounded once to fp32 and then to bf16: the epilogue reads bf16 gate/up
 *    ([P1] SwiGLU snippet) and L2 writes bf16 into the combine buffer
 *    ([P3] sections 4.2 and 5.1).  The fp64 accumulation below is exact for
 *    these operands (an e4m3 x e2m1 product has at most 6 significant bits).
 *  - Pool order inside an expert: ascending flat slot t*K+k (the pages
 *    allocate slots with atomics, [P3] section 3.1, so their order is not
 *    defined; a canonical order makes routing comparable bit for bit).
 *  - Combine: fp32 sum over ascending k of the valid slots, starting at +0,
 *    then bf16 round-to-nearest-even ([P1] "combine_utils.cuh" snippet;
 *    [P3] section 5.1).  A token with every slot masked gives +0.
 *  - Any negative expert index is a masked slot ([P3] section 4.1); an index
 *    >= E is rejected.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* bf16: the top half of an IEEE binary32.                                   */
/* ------------------------------------------------------------------------ */
float oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round to nearest, ties to even: keep the top 16 bits, look at the 16 bits
 * dropped. */
uint16_t oracle_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xFFFFu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

/* ------------------------------------------------------------------------ */
/* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities;  */
/* S.1111.111 is NaN; largest finite 448 = 1.75 * 2^8; subnormal step 2^-9.  */
/* ------------------------------------------------------------------------ */
float oracle_e4m3_to_f32(uint8_t code) {
    int sign = code >> 7;
    int ex = (code >> 3) & 0xF;
    int man = code & 7;
    double v;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0)
        v = ldexp((double)man, -9);
    else
        v = ldexp((double)(8 + man), ex - 10);
    return (float)(sign ? -v : v);
}

/* Round an exact real value to the nearest e4m3 value, ties to the even
 * code, saturating at +-448.  The quantum (spacing) of e4m3 near |v| is
 * 2^(E-3) for a normal binade 2^E (E >= -6) and 2^-9 below 2^-6. */
uint8_t oracle_e4m3_from_f64(double v) {
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    int ex, E, qexp;
    double n, r;
    if (isnan(v)) return 0x7F;
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    if (a == 0.0) return sign;
    frexp(a, &ex);
    E = ex - 1; /* a in [2^E, 2^(E+1)) */
    qexp = (E < -6 ? -6 : E) - 3;
    n = nearbyint(ldexp(a, -qexp)); /* default rounding mode: ties to even */
    r = ldexp(n, qexp);
    if (r == 0.0) return sign;
    frexp(r, &ex);
    E = ex - 1;
    if (E < -6) return (uint8_t)(sign | (uint8_t)ldexp(r, 9)); /* subnormal */
    return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | ((int)ldexp(r, 3 - E) - 8)));
}

void oracle_e4m3_from_f64_array(const double* v, uint8_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = oracle_e4m3_from_f64(v[i]);
}

/* ------------------------------------------------------------------------ */
/* OCP e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit.                    */
/* Magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.                      */
/* ------------------------------------------------------------------------ */
float oracle_e2m1_to_f32(uint8_t nibble) {
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float m = mag[nibble & 7];
    return (nibble & 8) ? -m : m;
}

/* ------------------------------------------------------------------------ */
/* UE8M0 scale byte b stands for 2^(b-127) (b = 255 is NaN, never produced). */
/* ------------------------------------------------------------------------ */
double oracle_ue8m0_value(uint8_t b) { return ldexp(1.0, (int)b - 127); }

/* Smallest b in [0, 254] with amax <= 448 * 2^(b-127).  The search starts
 * below the answer (amax >= 2^(ex-1) > 448 * 2^(ex-11)) and walks up. */
uint8_t oracle_ue8m0_for_e4m3(float amax) {
    double a = (double)amax;
    int ex, b;
    if (!(a > 0.0)) return 0;
    frexp(a, &ex);
    b = ex + 116;
    if (b < 0) b = 0;
    while (b < 254 && a > 448.0 * ldexp(1.0, b - 127)) ++b;
    return (uint8_t)b;
}

void oracle_ue8m0_for_e4m3_array(const float* amax, uint8_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = oracle_ue8m0_for_e4m3(amax[i]);
}

/* Quantise a row in groups of 32: amax -> scale byte -> e4m3 codes of the
 * value divided by the scale (a power of two, so the division is exact). */
int oracle_quant_e4m3_row(const float* v, int n, uint8_t* codes, uint8_t* scales) {
    if (n % 32) return -1;
    for (int g = 0; g < n / 32; ++g) {
        float amax = 0.0f;
        for (int j = 0; j < 32; ++j) {
            float a = fabsf(v[32 * g + j]);
            if (a > amax) amax = a;
        }
        uint8_t b = oracle_ue8m0_for_e4m3(amax);
        double inv = ldexp(1.0, 127 - (int)b);
        scales[g] = b;
        for (int j = 0; j < 32; ++j)
            codes[32 * g + j] = oracle_e4m3_from_f64((double)v[32 * g + j] * inv);
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* a1-a3: routing.  [P1] "dispatch.cuh" notify-warp snippet (per-expert      */
/* count, prefix sum); [P3] sections 3.1 and 8.3 (count, offsets, pool slot) */
/* and appendix A.2 (expert-major pool).                                     */
/* ------------------------------------------------------------------------ */
int oracle_route(int T, int K, int E, const int64_t* topk_idx, const float* topk_w,
                 int32_t* counts, int32_t* offsets, int32_t* pool_src,
                 int32_t* slot_to_pool, float* pool_w) {
    const int64_t TK = (int64_t)T * K;
    if (T < 0 || K < 1 || E < 1) return -1;
    for (int64_t f = 0; f < TK; ++f)
        if (topk_idx[f] >= E) return -5;

    /* a1: histogram of expert indices; negative = masked slot */
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t f = 0; f < TK; ++f)
        if (topk_idx[f] >= 0) counts[topk_idx[f]] += 1;

    /* a2: exclusive prefix sum, E+1 entries */
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];

    /* a3: pool row of slot f = offsets[e] + number of earlier slots with the
     * same expert; walking experts in order and slots in order inside each
     * expert produces exactly that numbering. */
    for (int64_t f = 0; f < TK; ++f) slot_to_pool[f] = -1;
    int32_t r = 0;
    for (int e = 0; e < E; ++e) {
        for (int64_t f = 0; f < TK; ++f) {
            if (topk_idx[f] != e) continue;
            pool_src[r] = (int32_t)f;
            slot_to_pool[f] = r;
            pool_w[r] = topk_w[f];
            ++r;
        }
    }
    return 0;
}

/* a4: dispatch = routing + a copy of each token row into the pool rows of its
 * valid slots, quantised to e4m3 per 32 columns (payload 0) or as bf16
 * (payload 1).  [P3] sections 3.1-3.2 (token rows pulled into the local
 * expert pool), appendix A.1 (FP8 token buffer with block scales). */
int oracle_dispatch(const oracle_shape_t* s, const uint16_t* x, const int64_t* topk_idx,
                    const float* topk_w, int payload, int32_t* counts, int32_t* offsets,
                    int32_t* pool_src, int32_t* slot_to_pool, float* pool_w,
                    void* pool, uint8_t* pool_scales) {
    const int T = s->T, H = s->H, K = s->K, E = s->E;
    int rc;
    if (H % 32) return -1;
    if (payload != 0 && payload != 1) return -1;
    rc = oracle_route(T, K, E, topk_idx, topk_w, counts, offsets, pool_src, slot_to_pool,
                      pool_w);
    if (rc) return rc;
    const int32_t R = offsets[E];
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : bad)
    for (int32_t r = 0; r < R; ++r) {
        const int64_t t = pool_src[r] / K;
        const uint16_t* xr = x + t * (int64_t)H;
        if (payload == 1) {
            memcpy((uint16_t*)pool + (int64_t)r * H, xr, (size_t)H * sizeof(uint16_t));
        } else {
            float* row = (float*)malloc((size_t)H * sizeof(float));
            if (!row) {
                bad |= 1;
                continue;
            }
            for (int h = 0; h < H; ++h) row[h] = oracle_bf16_to_f32(xr[h]);
            oracle_quant_e4m3_row(row, H, (uint8_t*)pool + (int64_t)r * H,
                                  pool_scales + (int64_t)r * (H / 32));
            free(row);
        }
    }
    return bad ? -3 : 0;
}

/* a9: combine.  [P1] "combine_utils.cuh" snippet (bf16 inputs, fp32 sums,
 * bf16 round-to-nearest out); [P3] section 5.1 (loop over top-k, masked
 * slots skipped, token-major output). */
int oracle_combine(int T, int K, int H, const uint16_t* o, const int32_t* slot_to_pool,
                   const float* topk_w, uint16_t* y) {
    if (T < 0 || K < 1 || H < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int h = 0; h < H; ++h) {
            float acc = 0.0f;
            for (int k = 0; k < K; ++k) {
                const int32_t r = slot_to_pool[(int64_t)t * K + k];
                if (r < 0) continue;
                float v = oracle_bf16_to_f32(o[(int64_t)r * H + h]);
                if (topk_w) v = v * topk_w[(int64_t)t * K + k];
                acc = acc + v;
            }
            y[(int64_t)t * H + h] = oracle_f32_to_bf16(acc);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-row building blocks of the expert MLP.                                */
/* ------------------------------------------------------------------------ */

/* Weight element (n, k) of one expert's [N][Kdim] FP4 matrix, dequantised:
 * e2m1 code times 2^(scale-127), scale per 32 along k.  Exact in double. */
static double w_deq(const uint8_t* Wq, const uint8_t* S, int Kdim, int64_t n, int k) {
    const uint8_t byte = Wq[(n * Kdim + k) / 2];
    const uint8_t nib = (k & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
    return (double)oracle_e2m1_to_f32(nib) * oracle_ue8m0_value(S[n * (Kdim / 32) + k / 32]);
}

/* One output element of a block-scaled GEMM row: the exact sum of the
 * products of the dequantised operands, rounded to fp32 then to bf16.
 * a5 / a8 ([P1] "complete compute pipeline" snippet, the UMMA step; [P3]
 * section 8.3). */
static uint16_t dot_bf16(const double* a_deq, const uint8_t* Wq, const uint8_t* S, int Kdim,
                         int64_t n) {
    double acc = 0.0;
    for (int k = 0; k < Kdim; ++k) acc += a_deq[k] * w_deq(Wq, S, Kdim, n, k);
    return oracle_f32_to_bf16((float)acc);
}

/* The same dot product with the weight row's scale looked up once per group
 * of 32 along k instead of once per element: every weight value, product
 * and partial sum is the same double as in dot_bf16 (e2m1 value times a
 * power of two is exact either way; the sum runs in the same ascending k
 * order), so the results are identical.  Used for the single-row entries. */
static uint16_t dot_bf16_grouped(const double* a_deq, const uint8_t* Wq, const uint8_t* S,
                                 int Kdim, int64_t n) {
    const uint8_t* wrow = Wq + n * (Kdim / 2);
    const uint8_t* srow = S + n * (Kdim / 32);
    double acc = 0.0;
    double val[16]; /* value of each e2m1 code under this group's scale */
    for (int g = 0; g < Kdim / 32; ++g) {
        const double sc = oracle_ue8m0_value(srow[g]);
        for (int c = 0; c < 16; ++c) val[c] = (double)oracle_e2m1_to_f32((uint8_t)c) * sc;
        for (int j = 0; j < 16; ++j) {
            const int k = 32 * g + 2 * j; /* byte j holds k (low nibble) and k + 1 */
            const uint8_t byte = wrow[k / 2];
            acc += a_deq[k] * val[byte & 0xF];
            acc += a_deq[k + 1] * val[byte >> 4];
        }
    }
    return oracle_f32_to_bf16((float)acc);
}

/* a6: SwiGLU scaled by the routing weight, fp32 throughout, in the pages'
 * order: e = exp(-g), d = 1 + e, s = g / d, a = (s * u) * w.  [P1] SwiGLU
 * snippet; [P3] section 4.2 (weight applied in the L1 epilogue). */
static float swiglu_w(uint16_t gate_bf16, uint16_t up_bf16, float w) {
    const float g = oracle_bf16_to_f32(gate_bf16);
    const float u = oracle_bf16_to_f32(up_bf16);
    const float e = expf(-g);
    const float d = 1.0f + e;
    const float s = g / d;
    const float su = s * u;
    return su * w;
}

/* L1 (a5), SwiGLU*w (a6) and requant (a7) of one routed row.  xq/xs: the
 * row's e4m3 codes and scales; w: its routing weight.  Writes the row's e4m3
 * activation codes aq[I] and scale bytes as[I/32]; h1_row[2I] (the bf16
 * gate|up) when not NULL.  par != 0 parallelises the output-column loop. */
static int l1_act_row(const oracle_shape_t* s, int e, const uint8_t* xq, const uint8_t* xs,
                      float w, const uint8_t* W1q, const uint8_t* S1, uint16_t* h1_row,
                      uint8_t* aq, uint8_t* as, int par, int grouped) {
    const int H = s->H, I = s->I;
    double* xd = (double*)malloc((size_t)H * sizeof(double));
    uint16_t* h1 = (uint16_t*)malloc((size_t)2 * I * sizeof(uint16_t));
    float* act = (float*)malloc((size_t)I * sizeof(float));
    if (!xd || !h1 || !act) {
        free(xd); free(h1); free(act);
        return -3;
    }
    const uint8_t* W1e = W1q + (int64_t)e * 2 * I * (H / 2);
    const uint8_t* S1e = S1 + (int64_t)e * 2 * I * (H / 32);

    /* dequantise the activation row (e4m3 code times its group scale) */
    for (int h = 0; h < H; ++h)
        xd[h] = (double)oracle_e4m3_to_f32(xq[h]) * oracle_ue8m0_value(xs[h / 32]);

    /* a5: L1, N = 2I columns: [0, I) gate, [I, 2I) up */
#pragma omp parallel for schedule(static) if (par)
    for (int n = 0; n < 2 * I; ++n)
        h1[n] = grouped ? dot_bf16_grouped(xd, W1e, S1e, H, n) : dot_bf16(xd, W1e, S1e, H, n);

    /* a6 + a7: SwiGLU * w, then e4m3 requant per 32 along I */
    for (int j = 0; j < I; ++j) act[j] = swiglu_w(h1[j], h1[I + j], w);
    oracle_quant_e4m3_row(act, I, aq, as);

    if (h1_row) memcpy(h1_row, h1, (size_t)2 * I * sizeof(uint16_t));
    free(xd); free(h1); free(act);
    return 0;
}

/* L2 (a8) of one activation row: K = I, N = H, unweighted, bf16 out.
 * aq/as: the row's e4m3 codes and scale bytes; writes o_row[H]. */
static int l2_row(const oracle_shape_t* s, int e, const uint8_t* aq, const uint8_t* as,
                  const uint8_t* W2q, const uint8_t* S2, uint16_t* o_row, int par, int grouped) {
    const int H = s->H, I = s->I;
    double* ad = (double*)malloc((size_t)I * sizeof(double));
    if (!ad) return -3;
    const uint8_t* W2e = W2q + (int64_t)e * H * (I / 2);
    const uint8_t* S2e = S2 + (int64_t)e * H * (I / 32);
    for (int i = 0; i < I; ++i)
        ad[i] = (double)oracle_e4m3_to_f32(aq[i]) * oracle_ue8m0_value(as[i / 32]);
#pragma omp parallel for schedule(static) if (par)
    for (int h = 0; h < H; ++h)
        o_row[h] = grouped ? dot_bf16_grouped(ad, W2e, S2e, I, h) : dot_bf16(ad, W2e, S2e, I, h);
    free(ad);
    return 0;
}

/* One routed row through the expert: L1 (a5), SwiGLU*w (a6), requant (a7),
 * L2 (a8).  xq/xs: the row's e4m3 codes and scales.  Writes the bf16 L2
 * row o_row[H]; optional h1_row[2I], aq_row[I], as_row[I/32].
 * par != 0 parallelises the output-column loops. */
static int expert_row(const oracle_shape_t* s, int e, const uint8_t* xq, const uint8_t* xs,
                      float w, const uint8_t* W1q, const uint8_t* S1, const uint8_t* W2q,
                      const uint8_t* S2, uint16_t* o_row, uint16_t* h1_row, uint8_t* aq_row,
                      uint8_t* as_row, int par) {
    const int I = s->I;
    uint8_t* aq = (uint8_t*)malloc((size_t)I);
    uint8_t* as = (uint8_t*)malloc((size_t)I / 32);
    int rc = -3;
    if (aq && as) {
        rc = l1_act_row(s, e, xq, xs, w, W1q, S1, h1_row, aq, as, par, 0);
        if (rc == 0) rc = l2_row(s, e, aq, as, W2q, S2, o_row, par, 0);
        if (rc == 0 && aq_row) memcpy(aq_row, aq, (size_t)I);
        if (rc == 0 && as_row) memcpy(as_row, as, (size_t)I / 32);
    }
    free(aq); free(as);
    return rc;
}

static int shape_ok(const oracle_shape_t* s) {
    return s && s->T >= 0 && s->H > 0 && s->I > 0 && s->E > 0 && s->K > 0 && s->H % 32 == 0 &&
           s->I % 32 == 0;
}

/* The whole layer, grouped: route, quantise into the expert-major pool, run
 * each pool row through its expert, combine.  [P1] "test_mega_moe.py"
 * snippet (the unfused five-step baseline) and [P3] sections 3-5. */
int oracle_forward(const oracle_shape_t* s, const uint16_t* x, const int64_t* topk_idx,
                   const float* topk_w, const uint8_t* W1q, const uint8_t* S1,
                   const uint8_t* W2q, const uint8_t* S2, uint16_t* y,
                   oracle_intermediates_t* mid) {
    if (!shape_ok(s)) return -1;
    const int T = s->T, H = s->H, I = s->I, E = s->E, K = s->K;
    const int64_t TK = (int64_t)T * K;
    if (T == 0) return 0;
    int32_t* counts = (int32_t*)malloc((size_t)E * sizeof(int32_t));
    int32_t* offsets = (int32_t*)malloc((size_t)(E + 1) * sizeof(int32_t));
    int32_t* pool_src = (int32_t*)malloc((size_t)TK * sizeof(int32_t));
    int32_t* slot_to_pool = (int32_t*)malloc((size_t)TK * sizeof(int32_t));
    float* pool_w = (float*)malloc((size_t)TK * sizeof(float));
    uint8_t* pool_q = (uint8_t*)malloc((size_t)TK * H);
    uint8_t* pool_s = (uint8_t*)malloc((size_t)TK * (H / 32));
    uint16_t* o = (uint16_t*)malloc((size_t)TK * H * sizeof(uint16_t));
    int rc = -3;
    if (!counts || !offsets || !pool_src || !slot_to_pool || !pool_w || !pool_q || !pool_s || !o)
        goto done;

    /* a1-a4 */
    rc = oracle_dispatch(s, x, topk_idx, topk_w, 0, counts, offsets, pool_src, slot_to_pool,
                         pool_w, pool_q, pool_s);
    if (rc) goto done;
    const int32_t R = offsets[E];

    /* a5-a8, one pool row at a time (rows are independent) */
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int32_t r = 0; r < R; ++r) {
        int e = 0;
        while (r >= offsets[e + 1]) ++e;
        bad |= expert_row(s, e, pool_q + (int64_t)r * H, pool_s + (int64_t)r * (H / 32),
                          pool_w[r], W1q, S1, W2q, S2, o + (int64_t)r * H,
                          mid && mid->h1 ? mid->h1 + (int64_t)r * 2 * I : NULL,
                          mid && mid->act_q ? mid->act_q + (int64_t)r * I : NULL,
                          mid && mid->act_s ? mid->act_s + (int64_t)r * (I / 32) : NULL, 0) != 0;
    }
    if (bad) {
        rc = -3;
        goto done;
    }

    /* a9 */
    rc = oracle_combine(T, K, H, o, slot_to_pool, NULL, y);

    if (mid) {
        if (mid->pool_q) memcpy(mid->pool_q, pool_q, (size_t)R * H);
        if (mid->pool_s) memcpy(mid->pool_s, pool_s, (size_t)R * (H / 32));
        if (mid->o) memcpy(mid->o, o, (size_t)R * H * sizeof(uint16_t));
        if (mid->counts) memcpy(mid->counts, counts, (size_t)E * sizeof(int32_t));
        if (mid->offsets) memcpy(mid->offsets, offsets, (size_t)(E + 1) * sizeof(int32_t));
        if (mid->pool_src) memcpy(mid->pool_src, pool_src, (size_t)R * sizeof(int32_t));
        if (mid->slot_to_pool) memcpy(mid->slot_to_pool, slot_to_pool, (size_t)TK * sizeof(int32_t));
        if (mid->pool_w) memcpy(mid->pool_w, pool_w, (size_t)R * sizeof(float));
    }
done:
    free(counts); free(offsets); free(pool_src); free(slot_to_pool); free(pool_w);
    free(pool_q); free(pool_s); free(o);
    return rc;
}

/* The same layer with no routing tables: each listed token, each valid slot
 * in ascending k, through its expert; then the fp32 sum of the slots. */
int oracle_forward_tokens(const oracle_shape_t* s, const uint16_t* x,
                          const int64_t* topk_idx, const float* topk_w,
                          const uint8_t* W1q, const uint8_t* S1, const uint8_t* W2q,
                          const uint8_t* S2, int n_tokens, const int32_t* tokens,
                          uint16_t* y_rows, uint8_t* aq_slots, uint8_t* as_slots) {
    if (!shape_ok(s) || n_tokens < 0) return -1;
    const int T = s->T, H = s->H, E = s->E, K = s->K;
    float* xrow = (float*)malloc((size_t)H * sizeof(float));
    uint8_t* xq = (uint8_t*)malloc((size_t)H);
    uint8_t* xs = (uint8_t*)malloc((size_t)H / 32);
    uint16_t* orow = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
    float* acc = (float*)malloc((size_t)H * sizeof(float));
    int rc = 0;
    if (!xrow || !xq || !xs || !orow || !acc) rc = -3;
    for (int i = 0; i < n_tokens && rc == 0; ++i) {
        const int t = tokens[i];
        if (t < 0 || t >= T) {
            rc = -1;
            break;
        }
        for (int h = 0; h < H; ++h) xrow[h] = oracle_bf16_to_f32(x[(int64_t)t * H + h]);
        oracle_quant_e4m3_row(xrow, H, xq, xs);
        for (int h = 0; h < H; ++h) acc[h] = 0.0f;
        for (int k = 0; k < K; ++k) {
            const int64_t e = topk_idx[(int64_t)t * K + k];
            if (e >= E) {
                rc = -5;
                break;
            }
            if (e < 0) continue;
            const int64_t slot = (int64_t)i * K + k;
            rc = expert_row(s, (int)e, xq, xs, topk_w[(int64_t)t * K + k], W1q, S1, W2q, S2, orow,
                            NULL, aq_slots ? aq_slots + slot * s->I : NULL,
                            as_slots ? as_slots + slot * (s->I / 32) : NULL, 1);
            if (rc) break;
            for (int h = 0; h < H; ++h) acc[h] = acc[h] + oracle_bf16_to_f32(orow[h]);
        }
        for (int h = 0; h < H; ++h) y_rows[(int64_t)i * H + h] = oracle_f32_to_bf16(acc[h]);
    }
    free(xrow); free(xq); free(xs); free(orow); free(acc);
    return rc;
}

/* Single routed rows, for checking chosen rows of a large layer: row i is
 * token tokens[i] of x through expert experts[i] with routing weight
 * weights[i] -- the same quantise -> L1 -> SwiGLU*w -> requant steps as the
 * grouped and per-token paths (a4-a7).  Writes aq_rows [n][I], as_rows
 * [n][I/32] and, when not NULL, h1_rows [n][2I]. */
int oracle_l1_act_rows(const oracle_shape_t* s, const uint16_t* x, const uint8_t* W1q,
                       const uint8_t* S1, int n, const int32_t* experts, const int32_t* tokens,
                       const float* weights, uint16_t* h1_rows, uint8_t* aq_rows,
                       uint8_t* as_rows) {
    if (!shape_ok(s) || n < 0) return -1;
    const int T = s->T, H = s->H, I = s->I, E = s->E;
    for (int i = 0; i < n; ++i)
        if (tokens[i] < 0 || tokens[i] >= T || experts[i] < 0 || experts[i] >= E) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < n; ++i) {
        float* xrow = (float*)malloc((size_t)H * sizeof(float));
        uint8_t* xq = (uint8_t*)malloc((size_t)H);
        uint8_t* xs = (uint8_t*)malloc((size_t)H / 32);
        if (!xrow || !xq || !xs) {
            bad |= 1;
        } else {
            for (int h = 0; h < H; ++h) xrow[h] = oracle_bf16_to_f32(x[(int64_t)tokens[i] * H + h]);
            oracle_quant_e4m3_row(xrow, H, xq, xs);
            bad |= l1_act_row(s, experts[i], xq, xs, weights[i], W1q, S1,
                              h1_rows ? h1_rows + (int64_t)i * 2 * I : NULL,
                              aq_rows + (int64_t)i * I, as_rows + (int64_t)i * (I / 32), 0, 1) != 0;
        }
        free(xrow); free(xq); free(xs);
    }
    return bad ? -3 : 0;
}

/* L2 (a8) alone on given activation rows: row i is the e4m3 codes
 * aq_rows[i] with scale bytes as_rows[i] through expert experts[i] ->
 * o_rows [n][H] bf16.  Lets a test feed the activations a GPU produced into
 * the exact L2, so that L2 is checked apart from the rounding of L1. */
int oracle_l2_rows(const oracle_shape_t* s, const uint8_t* W2q, const uint8_t* S2, int n,
                   const int32_t* experts, const uint8_t* aq_rows, const uint8_t* as_rows,
                   uint16_t* o_rows) {
    if (!shape_ok(s) || n < 0) return -1;
    const int H = s->H, I = s->I, E = s->E;
    for (int i = 0; i < n; ++i)
        if (experts[i] < 0 || experts[i] >= E) return -1;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int i = 0; i < n; ++i)
        bad |= l2_row(s, experts[i], aq_rows + (int64_t)i * I, as_rows + (int64_t)i * (I / 32), W2q,
                      S2, o_rows + (int64_t)i * H, 0, 1) != 0;
    return bad ? -3 : 0;
}
