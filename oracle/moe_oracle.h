/*
 * moe_oracle.h -- CPU oracle for one MoE layer's data-parallel hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, deliberately obvious
 * reference implementation.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant with the HIP library under combine_dispatch_amd/, and
 * neither side includes the other.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "DeepEP -> Mega MoE: the evolving boundary of communication and
 *        compute" (backyes.github.io/deepepv2, 07_deep_ep_10_evolution_to_megamoe)
 *        -- no numbered sections; cited by the code-snippet heading.
 *   [P2] "Normal vs Low-Latency: DeepEP's two communication philosophies
 *        mapped onto Mega MoE" (05_07_normal_vs_lowlatency), sections 1-12.
 *   [P3] "Dispatch/Combine in the DeepGEMM Mega MoE kernel"
 *        (05_01_dispatch_combine), sections 1-9 and appendix A.
 *
 * All pointers are host pointers.  Every function returns 0 on success and a
 * negative value on a bad argument (an expert index >= E, a shape that is
 * not a multiple of 32, ...).  Nothing is allocated for the caller.
 *
 * Numbers: bf16 values travel as uint16 bit patterns, e4m3 codes and UE8M0
 * scale bytes as uint8, FP4 e2m1 weights as two codes per byte (low nibble =
 * even K index).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t T; /* tokens */
    int32_t H; /* hidden size (L1 K, L2 N); multiple of 32 */
    int32_t I; /* intermediate size (L1 N = 2I, L2 K); multiple of 32 */
    int32_t E; /* experts */
    int32_t K; /* top-k slots per token */
} oracle_shape_t;

/* ---- element codecs (exported so tests can pin them) ------------------ */
float    oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f32_to_bf16(float f);            /* round to nearest even */
float    oracle_e4m3_to_f32(uint8_t code);       /* OCP e4m3fn */
uint8_t  oracle_e4m3_from_f64(double v);         /* RNE, saturating at 448 */
float    oracle_e2m1_to_f32(uint8_t nibble);     /* OCP e2m1 (low 4 bits) */
uint8_t  oracle_ue8m0_for_e4m3(float amax);      /* smallest 2^(b-127) with amax <= 448*2^(b-127) */
double   oracle_ue8m0_value(uint8_t b);          /* 2^(b-127) */
void     oracle_e4m3_from_f64_array(const double* v, uint8_t* out, size_t n);
void     oracle_ue8m0_for_e4m3_array(const float* amax, uint8_t* out, size_t n);

/* Quantise n fp32 values (n % 32 == 0) in groups of 32: scale byte per
 * group by the rule above, then e4m3 codes of v * 2^(127-b). */
int oracle_quant_e4m3_row(const float* v, int n, uint8_t* codes, uint8_t* scales);

/* ---- a1-a3: routing ---------------------------------------------------
 * counts[E], offsets[E+1], pool_src[T*K], slot_to_pool[T*K], pool_w[T*K].
 * Only the first R = offsets[E] entries of pool_src / pool_w are written;
 * slot_to_pool is -1 for masked slots (topk_idx < 0). */
int oracle_route(int T, int K, int E, const int64_t* topk_idx, const float* topk_w,
                 int32_t* counts, int32_t* offsets, int32_t* pool_src,
                 int32_t* slot_to_pool, float* pool_w);

/* ---- a1-a4: dispatch ---------------------------------------------------
 * payload 0: pool = e4m3 codes [T*K][H] plus pool_scales [T*K][H/32];
 * payload 1: pool = bf16 copies [T*K][H] (pool_scales unused, may be NULL). */
int oracle_dispatch(const oracle_shape_t* s, const uint16_t* x, const int64_t* topk_idx,
                    const float* topk_w, int payload, int32_t* counts, int32_t* offsets,
                    int32_t* pool_src, int32_t* slot_to_pool, float* pool_w,
                    void* pool, uint8_t* pool_scales);

/* ---- a9: combine -------------------------------------------------------
 * y[t] = bf16( sum over k ascending of valid slots of [w *] fp32(o[row]) ).
 * topk_w may be NULL (unweighted, as in the fused layer). */
int oracle_combine(int T, int K, int H, const uint16_t* o, const int32_t* slot_to_pool,
                   const float* topk_w, uint16_t* y);

/* Optional intermediates of the grouped forward (any pointer may be NULL). */
typedef struct {
    uint8_t*  pool_q;  /* [T*K][H]     e4m3 */
    uint8_t*  pool_s;  /* [T*K][H/32]  ue8m0 */
    uint16_t* h1;      /* [T*K][2I]    bf16 gate|up */
    uint8_t*  act_q;   /* [T*K][I]     e4m3 */
    uint8_t*  act_s;   /* [T*K][I/32]  ue8m0 */
    uint16_t* o;       /* [T*K][H]     bf16 */
    int32_t*  counts;  /* [E] */
    int32_t*  offsets; /* [E+1] */
    int32_t*  pool_src;     /* [T*K] */
    int32_t*  slot_to_pool; /* [T*K] */
    float*    pool_w;       /* [T*K] */
} oracle_intermediates_t;

/* ---- a1-a9: the whole layer, grouped (expert-major) --------------------- */
int oracle_forward(const oracle_shape_t* s, const uint16_t* x, const int64_t* topk_idx,
                   const float* topk_w, const uint8_t* W1q, const uint8_t* S1,
                   const uint8_t* W2q, const uint8_t* S2, uint16_t* y,
                   oracle_intermediates_t* mid);

/* ---- the same layer, brute force: for each listed token, each valid slot
 * runs quantise -> L1 -> SwiGLU -> requant -> L2 on that one row, then the
 * slots are summed.  y_rows is [n_tokens][H].  aq_slots ([n_tokens][K][I]
 * e4m3 codes) and as_slots ([n_tokens][K][I/32] scale bytes), when not NULL,
 * receive each valid slot's requantised activation row (masked slots are left
 * as they are). */
int oracle_forward_tokens(const oracle_shape_t* s, const uint16_t* x,
                          const int64_t* topk_idx, const float* topk_w,
                          const uint8_t* W1q, const uint8_t* S1, const uint8_t* W2q,
                          const uint8_t* S2, int n_tokens, const int32_t* tokens,
                          uint16_t* y_rows, uint8_t* aq_slots, uint8_t* as_slots);

/* ---- single routed rows (for checking chosen rows of a large layer) ----
 * oracle_l1_act_rows: row i = token tokens[i] of x, quantised, through
 * expert experts[i]'s L1, SwiGLU * weights[i], e4m3 requant (a4-a7) ->
 * aq_rows [n][I], as_rows [n][I/32], optional h1_rows [n][2I] (bf16 gate|up).
 * oracle_l2_rows: L2 alone (a8) on given activation rows: aq_rows[i] /
 * as_rows[i] through expert experts[i] -> o_rows [n][H] bf16.
 * Both run the same per-row steps as oracle_forward; rows in parallel. */
int oracle_l1_act_rows(const oracle_shape_t* s, const uint16_t* x, const uint8_t* W1q,
                       const uint8_t* S1, int n, const int32_t* experts, const int32_t* tokens,
                       const float* weights, uint16_t* h1_rows, uint8_t* aq_rows,
                       uint8_t* as_rows);
int oracle_l2_rows(const oracle_shape_t* s, const uint8_t* W2q, const uint8_t* S2, int n,
                   const int32_t* experts, const uint8_t* aq_rows, const uint8_t* as_rows,
                   uint16_t* o_rows);

/* Threads the parallel loops use (OpenMP). */
int oracle_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
