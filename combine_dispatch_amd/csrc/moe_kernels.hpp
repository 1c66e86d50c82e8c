// moe_kernels.hpp -- kernel entry points and launch constants shared between
// the kernel sources and the host API.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Routing: one wave owns a segment of kSegSlots consecutive flat slots.
constexpr int kSegSlots = 256;
constexpr int kRouteWaves = 4;  // waves per routing block
constexpr int kRouteThreads = kRouteWaves * 64;

// Grouped GEMM tiling: 256 x 256 output tile per 256-thread workgroup,
// 128 K per main-loop step, three LDS stages filled by direct global->LDS
// loads two steps ahead.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 128;
constexpr int kGemmThreads = 256;
constexpr int kStageA = kBM * kBK;          // e4m3 bytes
constexpr int kStageB = kBN * kBK / 2;      // e2m1 bytes
constexpr int kStageSA = kBM * 4;           // 4 scale bytes per row per step
constexpr int kStageSB = kBN * 4;
constexpr int kStageBytes = kStageA + kStageB + kStageSA + kStageSB;
constexpr int kStages = 3;

struct MTile {
    int32_t expert, row0, nrows, pad;
};

// Tile-per-workgroup GEMMs (batches whose experts hold few rows, and short
// reductions): tiles of at most 64 * RM rows (RM = 1 or 2) x 256 columns, one
// workgroup per tile and n-tile, dec_stages(RM) LDS stages of
// dec_stage_bytes(RM) each, so that two workgroups fit one CU.
constexpr int kDecRows = 64;
constexpr int kDecWorkgroupsPerCU = 2;
constexpr int dec_rows(int rm) { return kDecRows * rm; }
constexpr int dec_stage_a(int rm) { return dec_rows(rm) * kBK; }      // e4m3 rows
constexpr int kDecStageB = kBN * kBK / 2;                             // e2m1 rows
constexpr int dec_stage_sa(int rm) { return 4 * dec_rows(rm) * 4; }   // each wave's copy of the rows' scale words
constexpr int kDecStageSB = kBN * 4;
constexpr int dec_stage_bytes(int rm) { return dec_stage_a(rm) + kDecStageB + dec_stage_sa(rm) + kDecStageSB; }
constexpr int dec_stages(int rm) { return rm == 1 ? 3 : 2; }
static_assert(kDecWorkgroupsPerCU * dec_stages(1) * dec_stage_bytes(1) <= 160 * 1024, "LDS");
static_assert(kDecWorkgroupsPerCU * dec_stages(2) * dec_stage_bytes(2) <= 160 * 1024, "LDS");

// L1 and L2 in one launch: one workgroup per m-tile of at most kFusedRows
// rows (the second tile table, written with kFusedRows-row tiles), which
// keeps the tile's e4m3 activations (I <= kFusedMaxI columns) and their scale
// words in LDS between the two GEMMs.
constexpr int kFusedRows = 128;
constexpr int kFusedMaxI = 768;

// Tile records a persistent GEMM workgroup keeps in LDS: the launch must give
// no workgroup more tiles than this (at most ceil(ceil(tiles / 8) / (grid / 8))).
constexpr int kTileCache = 256;

// Block scales in "packed k-major" layout: one 4-byte word holds the UE8M0
// bytes of the 4 consecutive 32-wide k-blocks of one 128-wide K step w, in
// byte order (4w, 4w+2, 4w+1, 4w+3), and the words of one K step are stored
// contiguously over rows: word (w, row) at byte 4 * (w * rows_total + row).
struct GemmArgs {
    const uint8_t* A;    // e4m3 [rows][Kdim]; L1: token rows [T][Kdim] (see pool_tok)
    const uint8_t* SA;   // packed k-major words [Kdim/128][cap rows]
    const uint8_t* B;    // e2m1x2 [E][N][Kdim/2], or with b_tiled the tile-blocked layout below
    const uint8_t* SB;   // packed k-major words per expert [E][Kdim/128][N]
    int64_t sa_step;     // bytes between K steps of SA (4 * cap)
    // L1: pool row r takes A row pool_tok[r] (entries past the routed rows may
    // hold anything: they are clamped to T-1)
    const int32_t* pool_tok;
    int32_t T;
    const MTile* mtiles;
    const int32_t* num_mtiles;
    int32_t Kdim;        // reduction size
    int32_t N;           // output columns per expert of B (L1: 2I, L2: H)
    int32_t ntiles;      // workgroup tiles along N
    // L1 epilogue
    const float* pool_w; // [rows]
    uint8_t* act_q;      // e4m3 [rows][I]
    uint8_t* act_s;      // packed k-major words [I/128][cap], step act_s_step
    int64_t act_s_step;  // 4 * cap
    int32_t I;
    int32_t fast_math;
    int32_t sa_by_token;  // decode L1: SA = token-major words [T][Kdim/128], read by pool_tok
    // B codes tile-blocked (moe_pack_weights): for expert e, n-tile nt and K
    // step k one contiguous block of 256 rows x 64 bytes at
    // ((e * ntiles + nt) * (Kdim/128) + k) * 16384, row r of the block being
    // weight row 256 nt + r (L2) or, for L1, gate row 128 nt + r (r < 128)
    // and up row I + 128 nt + r - 128 (r >= 128)
    int32_t b_tiled;
    // L2 epilogue
    uint16_t* out;       // bf16 [rows][N]
};

__global__ void k_route_count(const int64_t* __restrict__ topk_idx, int64_t TK, int E,
                              int32_t* __restrict__ seg_hist, int32_t* __restrict__ seg_err,
                              int32_t* __restrict__ blk_hist, int32_t* __restrict__ blk_err);
// One-launch routing (see route.hip); used while nblk * E <= kRouteFusedMax,
// since every block reads all nblk rows of the block histograms.
constexpr int64_t kRouteFusedMax = 1 << 16;
inline size_t route_lds_bytes(int E) { return sizeof(int32_t) * 8 * (size_t)E + 8 * kRouteWaves * kSegSlots; }
__global__ void k_route(const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
                        int64_t TK, int E, int nbits, int K, const int32_t* __restrict__ blk_hist,
                        const int32_t* __restrict__ blk_err, int nblk, int32_t* __restrict__ counts,
                        int32_t* __restrict__ offsets, MTile* __restrict__ mtiles,
                        int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag,
                        int32_t* __restrict__ pool_src, int32_t* __restrict__ slot_to_pool,
                        float* __restrict__ pool_w, int32_t* __restrict__ pool_tok,
                        const uint32_t* __restrict__ tok_s, int W, int64_t cap,
                        uint32_t* __restrict__ pool_s, MTile* __restrict__ mtiles64,
                        int32_t* __restrict__ num_mtiles64, int dec_rows);
__global__ void k_route_scan(const int32_t* __restrict__ seg_hist,
                             const int32_t* __restrict__ seg_err, int nseg, int E,
                             int32_t* __restrict__ seg_base, int32_t* __restrict__ counts,
                             int32_t* __restrict__ offsets, MTile* __restrict__ mtiles,
                             int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag);
__global__ void k_route_scatter(const int64_t* __restrict__ topk_idx,
                                const float* __restrict__ topk_w, int64_t TK, int E, int nbits,
                                int K, const int32_t* __restrict__ seg_base,
                                int32_t* __restrict__ pool_src,
                                int32_t* __restrict__ slot_to_pool, float* __restrict__ pool_w,
                                int32_t* __restrict__ pool_tok);
__global__ void k_dispatch_fp8(const uint16_t* __restrict__ x, int64_t T, int H, int K, int tpb,
                               const int32_t* __restrict__ slot_to_pool, uint8_t* __restrict__ pool,
                               uint8_t* __restrict__ pool_s, uint8_t* __restrict__ tok_s);
__global__ void k_quantise_count(const uint16_t* __restrict__ x, int64_t T, int H, int tpb,
                                 uint8_t* __restrict__ x_q, uint8_t* __restrict__ tok_s,
                                 const int64_t* __restrict__ topk_idx, int64_t TK, int E, int ncount,
                                 int32_t* __restrict__ seg_hist, int32_t* __restrict__ seg_err,
                                 int32_t* __restrict__ blk_hist, int32_t* __restrict__ blk_err);
// a1-a4 in one launch for batches of at most kRouteWaves * kSegSlots slots
// (dynamic LDS: route_lds_bytes(E)): blocks [0, nroute = ceil(T*K / 256))
// route, the rest quantise.
constexpr int64_t kRouteSingleMax = (int64_t)kRouteWaves * kSegSlots;
__global__ void k_quantise_route(const uint16_t* __restrict__ x, int64_t T, int H, int tpb,
                                 uint8_t* __restrict__ x_q, uint8_t* __restrict__ tok_s,
                                 const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
                                 int64_t TK, int E, int nbits, int K, int nroute, int32_t* __restrict__ counts,
                                 int32_t* __restrict__ offsets, MTile* __restrict__ mtiles,
                                 int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag,
                                 int32_t* __restrict__ pool_src, int32_t* __restrict__ slot_to_pool,
                                 float* __restrict__ pool_w, int32_t* __restrict__ pool_tok,
                                 MTile* __restrict__ mtiles64, int32_t* __restrict__ num_mtiles64,
                                 int dec_rows);
__global__ void k_pool_scales(const uint32_t* __restrict__ tok_s, int W,
                              const int32_t* __restrict__ pool_tok,
                              const int32_t* __restrict__ offsets, int E, int64_t cap,
                              uint32_t* __restrict__ pool_s);
__global__ void k_scales_kmajor(const uint32_t* __restrict__ S, uint32_t* __restrict__ St, int N,
                                int W);
__global__ void k_dispatch_bf16(const uint16_t* __restrict__ x, int H, int K,
                                const int32_t* __restrict__ slot_to_pool,
                                uint16_t* __restrict__ pool);
// Tokens per dispatch / combine block: as many whole rows as fit 8192
// columns (at most kMaxBlockTokens), else one.
constexpr int kMaxBlockTokens = 32;
inline int tokens_per_block(int H) {
    const int t = 8192 / H;
    return t < 1 ? 1 : (t > kMaxBlockTokens ? kMaxBlockTokens : t);
}
// Blocks per group of tpb tokens: small batches split a block's columns
// into up to four pieces so that the grid covers the GPU.
inline int combine_parts(int64_t T, int H, int tpb) {
    const int64_t blocks = (T + tpb - 1) / tpb;
    if (blocks >= 1024) return 1;
    const int64_t by_cols = ((int64_t)tpb * H + 2047) / 2048;  // at least 2048 columns a piece
    return (int)(by_cols < 4 ? (by_cols < 1 ? 1 : by_cols) : 4);
}
__global__ void k_combine(const uint16_t* __restrict__ o, const int32_t* __restrict__ slot_to_pool,
                          const float* __restrict__ topk_w, int64_t T, int H, int K, int tpb, int nparts,
                          uint16_t* __restrict__ y);
// Weight codes [E][N][Kdim/2] -> the tile-blocked layout of GemmArgs.b_tiled
// (l1: the L1 weights' gate/up n-tiles, I the intermediate size; else L2).
constexpr int kBTileBytes = kBN * kBK / 2;
__global__ void k_pack_weights_tiled(const uint8_t* __restrict__ W, uint8_t* __restrict__ Wp, int E,
                                     int N, int Kdim, int I, int l1);
__global__ void k_gemm_l1(GemmArgs args);
// l1: the L1 GEMM's arguments (mtiles / num_mtiles: the kFusedRows-row
// table; act_q / act_s unused); l2: the L2 GEMM's B, SB, Kdim = I, N = H,
// ntiles = H / 256, out.
__global__ void k_gemm_fused(GemmArgs l1, GemmArgs l2);
__global__ void k_gemm_l2(GemmArgs args);
__global__ void k_gemm_l1_decode(GemmArgs args);
// the same for tile-blocked weights (b_tiled), whose blocks it streams with
// the non-temporal hint
__global__ void k_gemm_l1_decode_nt(GemmArgs args);
__global__ void k_gemm_l2_decode(GemmArgs args);
__global__ void k_gemm_l1_t128(GemmArgs args);
__global__ void k_gemm_l2_t128(GemmArgs args);

}  // namespace moe
