/*
 * moe_profile.h -- per-kernel timing of moe_fused_forward, for benchmarks.
 *
 * While profiling is on, every moe_fused_forward call records a HIP event on
 * its stream before its first launch and after each of its launches, so the
 * time between two consecutive events is one kernel's duration on the GPU
 * (plus the launch gap).  The events are timing-only (created without the
 * system-scope fence a default event performs when it is recorded, which
 * would add a gap of several microseconds before each launch).  Nothing is
 * synchronised until moe_profile_stop, which waits for the whole device.
 * Calls beyond max_calls are not recorded.  Not thread-safe: profile one
 * caller at a time.
 */
#ifndef MOE_PROFILE_H
#define MOE_PROFILE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Stages of moe_fused_forward, in launch order. */
enum {
    MOE_STAGE_WEIGHT_SCALES = 0, /* weight scales -> packed k-major words (canonical entry only) */
    MOE_STAGE_DISPATCH,        /* a4: e4m3 quantisation of the token rows; a1 per-segment
                                  expert histogram in the same launch (with at most 1024
                                  slots, T*K, all of a1-a3 in that launch) */
    MOE_STAGE_ROUTE_SCAN,      /* a2: offsets, segment bases, m-tile tables; in the one-launch
                                  routing (k_route) also a3; empty when the dispatch launch
                                  routed */
    MOE_STAGE_ROUTE_SCATTER,   /* a3: stable rank -> pool_src, slot_to_pool, pool_w, pool_tok
                                  (an empty interval when a3 ran in the one launch above) */
    MOE_STAGE_POOL_SCALES,     /* a4: the pool rows' scale words gathered by token (empty when
                                  the L1 GEMM reads them by token: the 64-row-tile GEMMs
                                  with at most 1024 routed slots) */
    MOE_STAGE_GEMM_L1,         /* a5-a7: L1 GEMM (gathers the token rows), SwiGLU*w, e4m3 requant;
                                  with gemm_tiles = MOE_TILES_FUSED also a8 (one launch) */
    MOE_STAGE_GEMM_L2,         /* a8: L2 GEMM, bf16 rows (empty with MOE_TILES_FUSED) */
    MOE_STAGE_COMBINE,         /* a9: top-k fp32 reduction to bf16 */
    MOE_PROFILE_STAGES
};

/* Start recording (creates MOE_PROFILE_STAGES + 1 events per call slot; host allocation only).
 * Returns 0, or MOE_ERR_INVALID_ARG for max_calls outside 1..4096, or
 * MOE_ERR_DEVICE if the events cannot be created. */
int moe_profile_start(int max_calls);

/* Stop, wait for the recorded events, and write the summed milliseconds of
 * each stage into stage_ms[MOE_PROFILE_STAGES] and the number of recorded
 * calls into *ncalls.  Returns 0, or MOE_ERR_INVALID_ARG if profiling was not
 * started, or MOE_ERR_DEVICE on an event error. */
int moe_profile_stop(double* stage_ms, int* ncalls);

/* Short name of a stage ("gemm_l1", ...), or "?" . */
const char* moe_profile_stage_name(int stage);

#ifdef __cplusplus
}
#endif
#endif
