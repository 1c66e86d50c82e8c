/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer library, libmoe_hip.so.
 *
 * One MoE layer's data-parallel hot path on one GPU: token dispatch into an
 * expert-major pool, the L1 grouped GEMM (FP8 e4m3 activations x FP4 e2m1
 * weights, one UE8M0 scale per 32 along K on both operands), SwiGLU scaled by
 * the routing weight and requantised to FP8, the L2 grouped GEMM, and the
 * fp32 top-k combine back to token-major bf16.
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "DeepEP -> Mega MoE: the evolving boundary of communication and
 *        compute" -- code-snippet headings, no numbered sections.
 *   [P2] "Normal vs Low-Latency: DeepEP's two communication philosophies
 *        mapped onto Mega MoE", sections 1-12.
 *   [P3] "Dispatch/Combine in the DeepGEMM Mega MoE kernel", sections 1-9,
 *        appendix A.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers, row-major, densely packed.  The
 *     caller owns every buffer; the library never allocates.
 *   - Calls are asynchronous on `stream` (NULL = the default stream) and never
 *     synchronise the host, except moe_options_t.debug_validate.
 *   - Return MOE_OK (0) or a negative status.  Shape, pointer and workspace
 *     errors are found on the host before anything is launched; a failed
 *     launch returns MOE_ERR_DEVICE.  Faults inside a kernel surface at the
 *     caller's next synchronisation, as usual for HIP.
 *   - T == 0 is valid and launches nothing.
 *   - Expert indices: a negative value marks a masked slot ([P3] section 4.1).
 *     An index >= E is a caller error: the kernels treat it as masked (they
 *     never index out of bounds with it) and raise a device flag that
 *     debug_validate turns into MOE_ERR_BAD_ROUTING.
 *
 * Number formats: bf16 = the top 16 bits of an IEEE binary32; e4m3 = OCP
 * e4m3fn bytes; e2m1 = OCP FP4, two codes per byte, the even K index in the
 * low nibble; ue8m0 = a scale byte b standing for 2^(b-127).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* a hipStream_t */

typedef struct {
    int32_t T; /* tokens, >= 0 */
    int32_t H; /* hidden size: L1 K and L2 N; multiple of 256 */
    int32_t I; /* intermediate size: L1 N = 2I (gate | up), L2 K; multiple of 128 */
    int32_t E; /* experts on this GPU, 1..1024 */
    int32_t K; /* top-k slots per token, 1..64 */
} moe_shape_t;

typedef struct {
    int32_t fast_math;        /* 1 (default): hardware exp and reciprocal in SwiGLU;
                                 0: library expf and IEEE division */
    float activation_clamp;   /* NaN (default) = none; any other value -> MOE_ERR_UNSUPPORTED */
    int32_t debug_validate;   /* 1: synchronise after routing and return
                                 MOE_ERR_BAD_ROUTING if an expert index was >= E */
    int32_t gemm_tiles;       /* which grouped-GEMM kernels run (same results
                                 up to the summation order inside each MFMA
                                 block, which all of them share):
                                 MOE_TILES_AUTO (default): chosen by shape;
                                 MOE_TILES_PERSISTENT: 256-row tiles, one
                                 workgroup per CU working through its tiles;
                                 MOE_TILES_64 / MOE_TILES_128: 64- or 128-row
                                 tiles, one workgroup each;
                                 MOE_TILES_FUSED: L1 and L2 in one launch, one
                                 workgroup per 128-row tile keeping the tile's
                                 e4m3 activations and their scales in LDS
                                 between the two GEMMs ([P1] "L1 Epilogue"
                                 snippet: the SwiGLU output stays in shared
                                 memory as the L2 input); needs I <= 768, and
                                 the workspace's act_q / act_s views are then
                                 not written.  The last three need the
                                 one-launch routing (ceil(T*K/1024) * E <=
                                 65536), else MOE_ERR_UNSUPPORTED; any other
                                 value -> MOE_ERR_INVALID_ARG */
} moe_options_t;

enum {
    MOE_TILES_AUTO = 0,
    MOE_TILES_PERSISTENT = 1,
    MOE_TILES_64 = 2,
    MOE_TILES_128 = 3,
    MOE_TILES_FUSED = 4
};

enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, negative size, unknown payload */
    MOE_ERR_UNSUPPORTED = -2, /* shape outside the kernels' tiling, option not implemented */
    MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
    MOE_ERR_DEVICE = -4,      /* not a gfx950 device, or a launch failed */
    MOE_ERR_BAD_ROUTING = -5, /* debug_validate found an expert index >= E */
    MOE_ERR_TOO_LARGE = -6    /* moe_fused_forward_packed_noalloc: the shape's workspace
                                 exceeds MOE_NOALLOC_SCRATCH_BYTES */
};

enum { MOE_PAYLOAD_FP8_E4M3 = 0, MOE_PAYLOAD_BF16 = 1 };

/* Defaults: fast_math 1, activation_clamp NaN, debug_validate 0. */
moe_options_t moe_default_options(void);

/* Bytes of device workspace moe_fused_forward needs for shape *s (capacity
 * T*K routed rows plus tile padding).  Host only; 0 on a shape that
 * moe_fused_forward would refuse (H % 256, I % 128, T * H >= 2^32, or the
 * basic limits). */
size_t moe_workspace_bytes(const moe_shape_t* s);

/* Bytes of device workspace moe_dispatch needs (routing scratch only). */
size_t moe_dispatch_workspace_bytes(const moe_shape_t* s);

/*
 * The whole layer, y = combine(L2(requant(SwiGLU(L1(dispatch(x))) * w))).
 * Steps: [P3] sections 3-5 (dispatch warps, L1 epilogue with SwiGLU and the
 * routing weight, L2, combine); [P1] "complete compute pipeline" snippet
 * (GEMM, SwiGLU, amax, FP8 requant, top-k reduction); the layer's entry with
 * y first and a caller-allocated buffer, [P2] section 2.
 *
 *   x         bf16  [T][H]
 *   topk_idx  int64 [T][K]   expert per slot; < 0 masked
 *   topk_w    fp32  [T][K]   routing weights (applied to the SwiGLU output)
 *   W1q       e2m1x2 [E][2I][H/2]  rows 0..I-1 gate, I..2I-1 up
 *   S1        ue8m0 [E][2I][H/32]  (4-byte aligned)
 *   W2q       e2m1x2 [E][H][I/2]
 *   S2        ue8m0 [E][H][I/32]   (4-byte aligned)
 *   y         bf16  [T][H], fully overwritten (an all-masked token gives +0)
 *   workspace device buffer of at least moe_workspace_bytes(s) bytes, 256-byte
 *             aligned; its contents on entry do not matter.
 * Numerics: x is quantised per token row in groups of 32 (scale = smallest
 * power of two with amax <= 448 * scale, e4m3 round-to-nearest-even); GEMM
 * outputs are fp32 sums rounded to bf16; SwiGLU is silu(gate) * up * w in
 * fp32, requantised the same way per 32 along I; combine sums the slots' bf16
 * rows in fp32 in ascending k, then rounds to bf16.
 * Shapes: H % 256 == 0, I % 128 == 0, 1 <= E <= 1024, 1 <= K <= 64,
 * T * K < 2^31, T * H < 2^32.  Otherwise MOE_ERR_UNSUPPORTED.
 */
int moe_fused_forward(const moe_shape_t* s, const moe_options_t* opt /* NULL = defaults */,
                      const void* x, const int64_t* topk_idx, const float* topk_w,
                      const uint8_t* W1q, const uint8_t* S1, const uint8_t* W2q,
                      const uint8_t* S2, void* y, void* workspace, size_t workspace_bytes,
                      moe_stream_t stream);

/*
 * Weight scales laid out once for many forward calls.  The pages' fused entry
 * takes its L1 and L2 weights already transformed into the kernel's own
 * layout ([P1] "tests/test_mega_moe.py" snippet, the fused call); here the
 * FP4 codes stay as given and only the scales are re-laid: for each expert and
 * each 128-wide K step, one 4-byte word per weight row holding the UE8M0 bytes
 * of the step's four 32-wide k-blocks in the order (0, 2, 1, 3), the words of
 * one step contiguous over rows.  The packed buffer holds S1's words, then,
 * from the next 256-byte boundary, S2's.  moe_fused_forward does the same
 * relayout into its workspace on every call.
 *
 * moe_packed_scales_bytes: bytes of that buffer for shape *s (host only; 0 on
 * a bad or unsupported shape).
 * moe_pack_weight_scales: fills `packed` (device, 256-byte aligned, at least
 * moe_packed_scales_bytes(s) bytes, owned by the caller) from S1 and S2 (as in
 * moe_fused_forward, 4-byte aligned).  Asynchronous on `stream`.  Errors as
 * moe_fused_forward; a short buffer gives MOE_ERR_WORKSPACE.
 * moe_fused_forward_packed: moe_fused_forward with the scales read from a
 * buffer that moe_pack_weight_scales filled for the same shape and weights;
 * the result is bit-identical.  The buffer must stay unchanged while calls
 * that read it are in flight.
 */
size_t moe_packed_scales_bytes(const moe_shape_t* s);
int moe_pack_weight_scales(const moe_shape_t* s, const uint8_t* S1, const uint8_t* S2,
                           void* packed, size_t packed_bytes, moe_stream_t stream);
int moe_fused_forward_packed(const moe_shape_t* s, const moe_options_t* opt /* NULL = defaults */,
                             const void* x, const int64_t* topk_idx, const float* topk_w,
                             const uint8_t* W1q, const uint8_t* W2q, const void* packed_scales,
                             void* y, void* workspace, size_t workspace_bytes,
                             moe_stream_t stream);

/*
 * Weights laid out once in the GEMMs' own layout, codes as well as scales
 * (the pages' fused entry takes both transformed: [P1] "tests/test_mega_moe.py"
 * snippet).  The FP4 codes are re-blocked so that what one GEMM K step of one
 * 256-row n-tile reads is one contiguous 16 KiB block: for expert e, n-tile
 * nt (L1: I/128 of them, each the 128 gate rows 128 nt.. and the 128 up rows
 * I + 128 nt..; L2: H/256, rows 256 nt..) and K step k (128 wide), block
 * ((e * ntiles + nt) * (K/128) + k) holds the tile's 256 rows in that order,
 * 64 bytes (128 codes) each.  A K step then reads one stretch of memory
 * instead of 256 rows a row-length apart.  Layout of the buffer: W1's blocks,
 * W2's blocks from the next 256-byte boundary, then from the next the packed
 * weight scales of moe_pack_weight_scales.
 *
 * moe_packed_weights_bytes: bytes of that buffer (host only; 0 on a bad or
 * unsupported shape) -- the size of the weights plus that of the packed scales.
 * moe_pack_weights: fills `packed` (device, 256-byte aligned, owned by the
 * caller) from W1q, W2q (16-byte aligned) and S1, S2 (4-byte aligned), as
 * given to moe_fused_forward.  Asynchronous on `stream`.  Errors as
 * moe_pack_weight_scales.
 * moe_fused_forward_prepacked: moe_fused_forward with every weight read from
 * that buffer (filled for the same shape); the result is bit-identical to
 * moe_fused_forward and moe_fused_forward_packed.  The buffer must stay
 * unchanged while calls that read it are in flight.
 */
size_t moe_packed_weights_bytes(const moe_shape_t* s);
int moe_pack_weights(const moe_shape_t* s, const uint8_t* W1q, const uint8_t* S1, const uint8_t* W2q,
                     const uint8_t* S2, void* packed, size_t packed_bytes, moe_stream_t stream);
int moe_fused_forward_prepacked(const moe_shape_t* s, const moe_options_t* opt /* NULL = defaults */,
                                const void* x, const int64_t* topk_idx, const float* topk_w,
                                const void* packed_weights, void* y, void* workspace,
                                size_t workspace_bytes, moe_stream_t stream);

/*
 * moe_fused_forward_packed without a workspace argument, for callers that
 * cannot allocate device memory around the call: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The
 * workspace is a device array inside the library, MOE_NOALLOC_SCRATCH_BYTES
 * (64 MiB) per GPU, which every GPU the library runs on holds until the
 * process ends; the call itself allocates nothing.  Inputs, outputs and the
 * packed weight scales are the caller's, as in moe_fused_forward_packed, and
 * the result is bit-identical to it.
 * Limit: shapes with moe_workspace_bytes(s) > MOE_NOALLOC_SCRATCH_BYTES get
 * MOE_ERR_TOO_LARGE before anything is launched (decode and small batches
 * fit: at H = 7168, I = 2048, E = 32 up to about 2000 routed rows T*K).
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (different streams, threads or processes' streams sharing the
 * library instance) race and give wrong results; calls ordered on one
 * stream are fine (the array's contents on entry do not matter).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_fused_forward_packed_noalloc(const moe_shape_t* s, const moe_options_t* opt /* NULL = defaults */,
                                     const void* x, const int64_t* topk_idx, const float* topk_w,
                                     const uint8_t* W1q, const uint8_t* W2q,
                                     const void* packed_scales, void* y, moe_stream_t stream);

/*
 * Dispatch only: routing metadata plus the expert-major pool.  [P3] sections
 * 3.1-3.2 and appendix A.2; [P1] "dispatch.cuh" snippets (per-expert count,
 * prefix sum, slot allocation, row copy).
 *   counts        int32 [E]     rows per expert
 *   offsets       int32 [E+1]   exclusive prefix sum; offsets[E] = R
 *   pool_src      int32 [T*K]   flat slot t*K+k of pool row r (first R entries)
 *   slot_to_pool  int32 [T*K]   pool row of slot t*K+k, -1 if masked
 *   pool_w        fp32  [T*K]   topk_w of pool row r (first R entries)
 *   pool          [T*K][H]      payload MOE_PAYLOAD_FP8_E4M3: e4m3 codes;
 *                               MOE_PAYLOAD_BF16: bf16 copies of x rows
 *   pool_scales   ue8m0 [T*K][H/32] (FP8 payload only; NULL for bf16)
 * Pool order is canonical: expert-major, and inside an expert ascending flat
 * slot t*K+k (the pages assign slots with atomics, so their order is not
 * fixed; this one is deterministic).  Rows past R are not written.
 * Shapes: H % 32 == 0 (H % 256 not required here), 1 <= E <= 1024.
 */
int moe_dispatch(const moe_shape_t* s, const void* x, const int64_t* topk_idx,
                 const float* topk_w, int payload, int32_t* counts, int32_t* offsets,
                 int32_t* pool_src, int32_t* slot_to_pool, float* pool_w, void* pool,
                 uint8_t* pool_scales, void* workspace, size_t workspace_bytes,
                 moe_stream_t stream);

/*
 * Combine only: y[t] = bf16( sum over k = 0..K-1 with slot_to_pool[t*K+k] >= 0
 * of [topk_w[t*K+k] *] fp32(pool_out[slot_to_pool[t*K+k]]) ), fp32 adds in
 * ascending k starting from +0.  [P1] "combine_utils.cuh" snippet; [P3]
 * section 5.1.  topk_w may be NULL (unweighted: the fused layer applies the
 * weight before L2); with weights each product is rounded to fp32 before
 * the add.
 *   pool_out      bf16 [R][H] in pool order (R = rows referenced)
 *   slot_to_pool  int32 [T*K]
 *   y             bf16 [T][H]
 * Shapes: H % 8 == 0.
 */
int moe_combine(const moe_shape_t* s, const void* pool_out, const int32_t* slot_to_pool,
                const float* topk_w, void* y, moe_stream_t stream);

/* Byte offsets of intermediates inside a moe_fused_forward workspace, so that
 * tests can read them after a call (all -1 and MOE_ERR_INVALID_ARG on a shape
 * moe_fused_forward would refuse).
 * The fused layer quantises every token row once (x_q, token-major) and its
 * L1 GEMM reads pool row r from token row pool_tok[r]; the expert-major pool
 * itself is not materialised (moe_dispatch materialises it).
 * Block scales are stored as 4-byte words of four UE8M0 bytes, one word per
 * row and 128-column K step w, holding the row's 32-column groups 4w, 4w+2,
 * 4w+1, 4w+3 in that byte order (the pages' SF buffers pack 4 UE8M0 per 128
 * columns, [P3] appendix A.1): for x_s token-major, word (t, w) at byte
 * 4 * (t * H/128 + w); for pool_s and act_s packed k-major, word (r, w) at
 * byte 4 * (w * cap + r), so that one K step of a row tile is one contiguous
 * run. */
typedef struct {
    int64_t counts, offsets, pool_src, slot_to_pool, pool_w; /* routing arrays */
    int64_t pool_tok;         /* int32 [cap]: token of pool row r (first R entries) */
    int64_t x_q, x_s;         /* e4m3 [T][H], words [T][H/128] */
    int64_t pool_s;           /* x_s words of the pool rows, packed k-major [H/128][cap];
                                 not written when the call runs the 64-row-tile GEMMs (by
                                 default when T*K <= 64*E) with T*K <= 1024: their L1
                                 GEMM then reads x_s by token */
    int64_t act_q, act_s;     /* e4m3 [cap][I], packed k-major words [I/128][cap] */
    int64_t l2_out;           /* bf16 [cap][H] */
    int64_t capacity_rows;    /* cap = T*K + tile padding */
} moe_workspace_views_t;

int moe_workspace_views(const moe_shape_t* s, moe_workspace_views_t* v);

/* Human-readable text of a status code (static storage). */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif
