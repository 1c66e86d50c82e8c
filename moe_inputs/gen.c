/*
 * gen.c -- seeded synthetic inputs for the MoE layer (bulk tensors).
 *
 * This file prepares inputs only; it holds none of the layer's arithmetic.
 * Both the HIP library's tests/benchmark and the CPU oracle consume the bytes
 * it writes.
 *
 * Random numbers: Philox4x32-10, the counter-based generator of Salmon,
 * Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
 * (SC'11): ten rounds of two 32x32->64-bit multiplies with the round
 * multipliers 0xD2511F53 / 0xCD9E8D57 and a Weyl key schedule
 * (0x9E3779B9, 0xBB67AE85).  Element i of a stream uses counter block i/4
 * (words 0-1), the stream id in word 2, and the seed as the key; each
 * 4-word output gives four normals by the Box-Muller transform.
 *
 * Weights follow the workload recipe "N(0, std) values, FP4 e2m1 codes with
 * one power-of-two (UE8M0) scale per 32 along K": per group the scale is the
 * smallest power of two that fits the group's largest magnitude under 6, and
 * each value goes to the nearest e2m1 magnitude, ties to the even code.
 * Two codes per byte, the even K index in the low nibble.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -shared -fPIC -o libmoe_inputs.so gen.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef struct {
    uint32_t v[4];
} u32x4;

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
    uint64_t p = (uint64_t)a * (uint64_t)b;
    *hi = (uint32_t)(p >> 32);
    *lo = (uint32_t)p;
}

static u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
    for (int r = 0; r < 10; ++r) {
        uint32_t hi0, lo0, hi1, lo1;
        mulhilo(0xD2511F53u, c.v[0], &hi0, &lo0);
        mulhilo(0xCD9E8D57u, c.v[2], &hi1, &lo1);
        u32x4 n;
        n.v[0] = hi1 ^ c.v[1] ^ k0;
        n.v[1] = lo1;
        n.v[2] = hi0 ^ c.v[3] ^ k1;
        n.v[3] = lo0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

/* One Philox4x32-10 block: out = philox(ctr, key), for known-answer checks. */
void gen_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    u32x4 c = {{ctr[0], ctr[1], ctr[2], ctr[3]}};
    const u32x4 r = philox4x32_10(c, key[0], key[1]);
    memcpy(out, r.v, sizeof r.v);
}

/* Four N(0,1) doubles from counter block `blk` of stream `stream`. */
static void normals4(uint64_t seed, uint32_t stream, uint64_t blk, double out[4]) {
    u32x4 c = {{(uint32_t)blk, (uint32_t)(blk >> 32), stream, 0u}};
    u32x4 r = philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
    const double two_pi = 6.283185307179586476925286766559;
    for (int p = 0; p < 2; ++p) {
        double u1 = ((double)r.v[2 * p] + 0.5) * (1.0 / 4294967296.0);
        double u2 = ((double)r.v[2 * p + 1] + 0.5) * (1.0 / 4294967296.0);
        double rad = sqrt(-2.0 * log(u1));
        out[2 * p] = rad * cos(two_pi * u2);
        out[2 * p + 1] = rad * sin(two_pi * u2);
    }
}

/* out[i] = mean + std * N(0,1), as float32. */
void gen_normal_f32(uint64_t seed, uint32_t stream, double mean, double std, float* out,
                    int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < (n + 3) / 4; ++b) {
        double q[4];
        normals4(seed, stream, (uint64_t)b, q);
        for (int j = 0; j < 4 && 4 * b + j < n; ++j) out[4 * b + j] = (float)(mean + std * q[j]);
    }
}

/* N(0,1) as float32, then to bf16 bits by round-to-nearest-even. */
void gen_normal_bf16(uint64_t seed, uint32_t stream, uint16_t* out, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < (n + 3) / 4; ++b) {
        double q[4];
        normals4(seed, stream, (uint64_t)b, q);
        for (int j = 0; j < 4 && 4 * b + j < n; ++j) {
            float f = (float)q[j];
            uint32_t u;
            memcpy(&u, &f, 4);
            uint32_t lsb = (u >> 16) & 1u;
            out[4 * b + j] = (uint16_t)((u + 0x7FFFu + lsb) >> 16);
        }
    }
}

/* Nearest e2m1 code (0..7 magnitude, bit 3 sign) of a value already divided
 * by its group scale (|a| <= 6).  Midpoints between neighbours go to the even
 * code. */
static uint8_t nearest_e2m1(double v) {
    static const double mid[7] = {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0};
    double a = fabs(v);
    int code = 0;
    for (int i = 0; i < 7; ++i) {
        if (a > mid[i])
            code = i + 1;
        else if (a == mid[i])
            code = (i & 1) ? i + 1 : i;
    }
    if (code == 0) return 0; /* +0 for values that round to zero */
    return (uint8_t)(code | (v < 0 ? 8 : 0));
}

/* rows x kdim weights ~ N(0, std), quantised in groups of 32 along kdim.
 * q: [rows][kdim/2] packed codes; s: [rows][kdim/32] scale bytes.  Row r of
 * the stream starts at element r*kdim, so any row range can be regenerated
 * on its own. */
void gen_fp4_weights(uint64_t seed, uint32_t stream, double std, int64_t rows, int32_t kdim,
                     uint8_t* q, uint8_t* s) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[32];
        for (int g = 0; g < kdim / 32; ++g) {
            double amax = 0.0;
            /* kdim % 32 == 0, so a group starts on a 4-element counter block */
            for (int j = 0; j < 32; j += 4)
                normals4(seed, stream, (uint64_t)(r * kdim + 32 * g + j) >> 2, v + j);
            for (int j = 0; j < 32; ++j) {
                v[j] = (double)(float)(std * v[j]); /* the recipe draws fp32 weights */
                if (fabs(v[j]) > amax) amax = fabs(v[j]);
            }
            /* smallest b with amax <= 6 * 2^(b-127); start below it */
            int b = 0, ex = 0;
            if (amax > 0.0) {
                frexp(amax, &ex);
                b = ex + 123;
                if (b < 0) b = 0;
            }
            while (b < 254 && amax > 6.0 * ldexp(1.0, b - 127)) ++b;
            s[r * (kdim / 32) + g] = (uint8_t)b;
            for (int j = 0; j < 32; j += 2) {
                uint8_t lo = nearest_e2m1(ldexp(v[j], 127 - b));
                uint8_t hi = nearest_e2m1(ldexp(v[j + 1], 127 - b));
                q[r * (kdim / 2) + (32 * g + j) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}
