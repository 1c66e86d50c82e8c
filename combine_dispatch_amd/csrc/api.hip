// api.hip -- the C ABI declared in include/moe.h: argument checks, workspace
// carving and the launch sequence.  No allocation, no host synchronisation
// (except the opt-in debug validation).
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "../../include/moe_profile.h"
#include "moe_kernels.hpp"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    size_t seg_hist, seg_base, seg_err, blk_hist, blk_err, counts, offsets, mtiles, num_mtiles,
        err_flag, mtiles64, num_mtiles64;
    size_t pool_src, slot_to_pool, pool_w, pool_tok, x_q, pool_s, act_q, act_s, l2_out, s1t, s2t,
        tok_s;
    size_t routing_end;  // bytes moe_dispatch needs
    size_t total;
    int64_t cap;         // pool rows incl. tile padding
    int64_t nseg;
    int64_t max_mtiles;
    int64_t max_mtiles64;  // tiles of at most kDecRows rows
};

bool shape_basic_ok(const moe_shape_t* s) {
    return s && s->T >= 0 && s->H > 0 && s->I > 0 && s->E >= 1 && s->E <= 1024 && s->K >= 1 &&
           s->K <= 64 && (int64_t)s->T * s->K < (int64_t(1) << 31);
}

// Shapes the fused layer's GEMM tiling takes: H a multiple of the 256-column
// tile (L2 N) and of the 128-wide K step (L1 K), I a multiple of 128 (L1 N
// in gate/up halves of 128, L2 K step), and 32-bit token-row offsets.
bool fused_shape_ok(const moe_shape_t* s) {
    return shape_basic_ok(s) && s->H % kBN == 0 && s->I % 128 == 0 &&
           (int64_t)s->T * s->H < (int64_t(1) << 32);
}

// Workspace regions, in order.  The routing scratch comes first so that
// moe_dispatch can use a prefix of the same layout.
Layout make_layout(const moe_shape_t* s) {
    Layout L;
    const int64_t TK = (int64_t)s->T * s->K;
    const int64_t E = s->E;
    L.nseg = (TK + kSegSlots - 1) / kSegSlots;
    L.max_mtiles = TK / kBM + (E < TK ? E : TK) + 1;
    L.cap = TK + kBM;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.seg_hist = take(sizeof(int32_t) * L.nseg * E);
    L.seg_base = take(sizeof(int32_t) * L.nseg * E);
    L.seg_err = take(sizeof(int32_t) * (L.nseg + 1));
    const int64_t nblk = (L.nseg + kRouteWaves - 1) / kRouteWaves;
    L.blk_hist = take(sizeof(int32_t) * nblk * E);
    L.blk_err = take(sizeof(int32_t) * (nblk + 1));
    L.mtiles = take(sizeof(MTile) * L.max_mtiles);
    L.num_mtiles = take(sizeof(int32_t));
    L.err_flag = take(sizeof(int32_t));
    L.max_mtiles64 = TK / kDecRows + (E < TK ? E : TK) + 1;
    L.mtiles64 = take(sizeof(MTile) * L.max_mtiles64);
    L.num_mtiles64 = take(sizeof(int32_t));
    L.routing_end = o;
    L.counts = take(sizeof(int32_t) * E);
    L.offsets = take(sizeof(int32_t) * (E + 1));
    L.pool_src = take(sizeof(int32_t) * L.cap);
    L.slot_to_pool = take(sizeof(int32_t) * (TK + 1));
    L.pool_w = take(sizeof(float) * L.cap);
    L.pool_tok = take(sizeof(int32_t) * L.cap);
    L.x_q = take((size_t)s->T * s->H);
    L.pool_s = take((size_t)L.cap * (s->H / 32));
    L.act_q = take((size_t)L.cap * s->I);
    L.act_s = take((size_t)L.cap * (s->I / 32));
    L.l2_out = take((size_t)L.cap * s->H * 2);
    L.s1t = take((size_t)E * 2 * s->I * (s->H / 32));
    L.s2t = take((size_t)E * s->H * (s->I / 32));
    L.tok_s = take((size_t)s->T * (s->H / 32));
    L.total = o;
    return L;
}

// Packed weight scales (moe_pack_weight_scales): S1's words, then S2's.
size_t packed_s1_bytes(const moe_shape_t* s) { return (size_t)s->E * 2 * s->I * (s->H / 32); }
size_t packed_total_bytes(const moe_shape_t* s) {
    return align_up(packed_s1_bytes(s)) + (size_t)s->E * s->H * (s->I / 32);
}

// Tile-blocked weights (moe_pack_weights): W1's codes, W2's codes, then the
// packed weight scales, each from a 256-byte boundary.
size_t tiled_w1_bytes(const moe_shape_t* s) { return (size_t)s->E * 2 * s->I * (s->H / 2); }
size_t tiled_w2_bytes(const moe_shape_t* s) { return (size_t)s->E * s->H * (s->I / 2); }
size_t tiled_w2_offset(const moe_shape_t* s) { return align_up(tiled_w1_bytes(s)); }
size_t tiled_scales_offset(const moe_shape_t* s) { return tiled_w2_offset(s) + align_up(tiled_w2_bytes(s)); }
size_t tiled_total_bytes(const moe_shape_t* s) { return tiled_scales_offset(s) + packed_total_bytes(s); }

// Weight scales (ue8m0 [E][N][Kdim/32], rows of Kdim/128 words) -> the packed
// k-major words the GEMMs load per K step, for both layers.
void launch_pack_scales(const moe_shape_t* s, const uint8_t* S1, const uint8_t* S2, uint8_t* s1t,
                        uint8_t* s2t, hipStream_t stream) {
    const int H = s->H, I = s->I;
    hipLaunchKernelGGL(k_scales_kmajor, dim3(2 * I / 64, s->E, (H / 128 + 63) / 64), dim3(256), 0,
                       stream, reinterpret_cast<const uint32_t*>(S1), reinterpret_cast<uint32_t*>(s1t),
                       2 * I, H / 128);
    hipLaunchKernelGGL(k_scales_kmajor, dim3(H / 64, s->E, (I / 128 + 63) / 64), dim3(256), 0,
                       stream, reinterpret_cast<const uint32_t*>(S2), reinterpret_cast<uint32_t*>(s2t),
                       H, I / 128);
}

// gfx950 check, cached per device.
int device_ok() {
    static int cache[64];  // 0 unknown, 1 ok, 2 bad
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64 && cache[dev]) return cache[dev] == 1;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    const int ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) cache[dev] = ok ? 1 : 2;
    return ok;
}

// Workgroups of a persistent GEMM launch: one per CU (at most one fits, by
// LDS), a multiple of 8 so that every XCD gets the same number, no more than
// there can be tiles, and enough that no workgroup gets more than kTileCache
// tiles (workgroups beyond the CU count then wait for a free CU).
unsigned gemm_grid(int64_t max_tiles) {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int n = dev < 64 ? cus[dev] : 0;
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
            n = 8;
        if (dev < 64) cus[dev] = n;
    }
    int64_t w = n / 8 * 8;
    const int64_t need = (max_tiles + 7) / 8 * 8;
    if (need < w) w = need;
    const int64_t per_xcd = (max_tiles + 7) / 8;
    const int64_t min_w = 8 * ((per_xcd + kTileCache - 1) / kTileCache);
    if (w < min_w) w = min_w;
    return (unsigned)(w < 8 ? 8 : w);
}

int launch_status() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// ---- optional per-kernel timing (moe_profile.h) ------------------------------
struct Profile {
    bool on = false;
    int max_calls = 0;
    int ncalls = 0;
    std::vector<hipEvent_t> ev;  // (MOE_PROFILE_STAGES + 1) per call
};
Profile g_prof;
constexpr int kMarks = MOE_PROFILE_STAGES + 1;

// Slot of this call, or -1 when not profiling.
int prof_begin(hipStream_t stream) {
    if (!g_prof.on || g_prof.ncalls >= g_prof.max_calls) return -1;
    const int c = g_prof.ncalls++;
    (void)hipEventRecord(g_prof.ev[c * kMarks], stream);
    return c;
}

void prof_mark(int call, int stage, hipStream_t stream) {
    if (call >= 0) (void)hipEventRecord(g_prof.ev[call * kMarks + stage + 1], stream);
}

int bits_for(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b < 1 ? 1 : b;
}

// a1-a3 into caller-visible arrays; the routing scratch lives at ws.
int route_blocks(const Layout& L) { return (int)((L.nseg + kRouteWaves - 1) / kRouteWaves); }

// One-launch routing (k_route) while every block can afford to read all the
// block histograms; otherwise a single-block scan, then the scatter.
bool route_fused(const Layout& L, int E) { return (int64_t)route_blocks(L) * E <= kRouteFusedMax; }

// Which GEMM kernels a call runs.  rm = 0: both persistent over 256-row
// tiles; rm = 1: both tile-per-workgroup over 64-row tiles (at most 64
// routed slots per expert on average: the weights stream through once);
// rm = 2: 128-row tiles for l1 / l2 where set.  The tile-per-workgroup
// kernels read the second tile table, which the one-launch routing writes.
// fused: L1 and L2 in one launch over the 128-row table (rm = 2).
struct TilePlan {
    int rm;
    bool l1, l2;
    bool fused;
};
constexpr bool kT128L1 = false, kT128L2 = false;
TilePlan tile_plan(const moe_shape_t* s, const Layout& L, int choice) {
    const int64_t TK = (int64_t)s->T * s->K;
    if (choice == MOE_TILES_PERSISTENT || !route_fused(L, s->E)) return {0, false, false, false};
    if (choice == MOE_TILES_64) return {1, true, true, false};
    if (choice == MOE_TILES_128) return {2, true, true, false};
    if (choice == MOE_TILES_FUSED) return {kFusedRows / kDecRows, true, true, true};
    if (TK <= (int64_t)kDecRows * s->E) return {1, true, true, false};
    if (kT128L1 || kT128L2) return {2, kT128L1, kT128L2, false};
    return {0, false, false, false};
}

// a1 (unless the caller's first launch already counted: `counted`), a2, a3,
// and, with pool_s set, the pool rows' A-scale words gathered from the
// token words tok_s ([T][W]) into the GEMM's packed k-major layout.
int run_routing(const moe_shape_t* s, const Layout& L, const int64_t* topk_idx, const float* topk_w,
                uint8_t* ws, int32_t* pool_tok, int32_t* counts, int32_t* offsets, int32_t* pool_src,
                int32_t* slot_to_pool, float* pool_w, hipStream_t stream, bool counted, int pc,
                const uint32_t* tok_s, uint32_t* pool_s, int dec_rows = kDecRows) {
    const int64_t TK = (int64_t)s->T * s->K;
    const int E = s->E;
    const int nblk = route_blocks(L);
    const size_t lds = sizeof(int32_t) * kRouteWaves * E;
    int32_t* seg_hist = reinterpret_cast<int32_t*>(ws + L.seg_hist);
    int32_t* seg_base = reinterpret_cast<int32_t*>(ws + L.seg_base);
    int32_t* seg_err = reinterpret_cast<int32_t*>(ws + L.seg_err);
    int32_t* blk_hist = reinterpret_cast<int32_t*>(ws + L.blk_hist);
    int32_t* blk_err = reinterpret_cast<int32_t*>(ws + L.blk_err);
    const bool fused = route_fused(L, E);
    if (!counted && nblk > 0)
        hipLaunchKernelGGL(k_route_count, dim3(nblk), dim3(kRouteThreads), lds, stream, topk_idx,
                           TK, E, seg_hist, seg_err, fused ? blk_hist : static_cast<int32_t*>(nullptr),
                           blk_err);
    if (fused) {
        hipLaunchKernelGGL(k_route, dim3((unsigned)(nblk > 0 ? nblk : 1)), dim3(kRouteThreads),
                           route_lds_bytes(E), stream, topk_idx, topk_w, TK, E, bits_for(E), s->K,
                           blk_hist, blk_err, nblk, counts, offsets,
                           reinterpret_cast<MTile*>(ws + L.mtiles),
                           reinterpret_cast<int32_t*>(ws + L.num_mtiles),
                           reinterpret_cast<int32_t*>(ws + L.err_flag), pool_src, slot_to_pool, pool_w,
                           pool_tok, tok_s, s->H / 128, (int64_t)L.cap,
                           static_cast<uint32_t*>(nullptr), reinterpret_cast<MTile*>(ws + L.mtiles64),
                           reinterpret_cast<int32_t*>(ws + L.num_mtiles64), dec_rows);
        prof_mark(pc, MOE_STAGE_ROUTE_SCAN, stream);
        prof_mark(pc, MOE_STAGE_ROUTE_SCATTER, stream);
        // the scale words are a grid-wide copy (megabytes): a kernel of their own
        if (pool_s)
            hipLaunchKernelGGL(k_pool_scales, dim3((unsigned)((L.cap + 255) / 256)), dim3(256), 0,
                               stream, tok_s, s->H / 128, pool_tok, offsets, s->E, (int64_t)L.cap, pool_s);
        prof_mark(pc, MOE_STAGE_POOL_SCALES, stream);
        return launch_status();
    }
    const int scan_threads = 1024;  // several threads per expert split the segments
    hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(scan_threads), 0, stream, seg_hist, seg_err,
                       (int)L.nseg, E, seg_base, counts, offsets,
                       reinterpret_cast<MTile*>(ws + L.mtiles),
                       reinterpret_cast<int32_t*>(ws + L.num_mtiles),
                       reinterpret_cast<int32_t*>(ws + L.err_flag));
    prof_mark(pc, MOE_STAGE_ROUTE_SCAN, stream);
    if (nblk > 0)
        hipLaunchKernelGGL(k_route_scatter, dim3(nblk), dim3(kRouteThreads), lds, stream, topk_idx,
                           topk_w, TK, E, bits_for(E), s->K, seg_base, pool_src, slot_to_pool, pool_w,
                           pool_tok);
    prof_mark(pc, MOE_STAGE_ROUTE_SCATTER, stream);
    if (pool_s)
        hipLaunchKernelGGL(k_pool_scales, dim3((unsigned)((L.cap + 255) / 256)), dim3(256), 0,
                           stream, tok_s, s->H / 128, pool_tok, offsets, s->E, (int64_t)L.cap, pool_s);
    prof_mark(pc, MOE_STAGE_POOL_SCALES, stream);
    return launch_status();
}

int check_routing_flag(uint8_t* ws, const Layout& L, hipStream_t stream) {
    int32_t flag = 0;
    if (hipMemcpyAsync(&flag, ws + L.err_flag, sizeof flag, hipMemcpyDeviceToHost, stream) !=
            hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return MOE_ERR_DEVICE;
    return flag ? MOE_ERR_BAD_ROUTING : MOE_OK;
}

// ---- the allocation-free entry's workspace ---------------------------------
// A file-scope device array: every GPU the library runs on holds its own copy
// for the life of the process.  In host code `scratch` names a host-side
// stand-in, not device memory, so host code uses only the address that
// hipGetSymbolAddress returns for the current device (scratch_device_ptr).
constexpr size_t kNoAllocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void* scratch_device_ptr() {
    static std::mutex mu;
    static void* ptrs[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        ptrs[dev] = p;
    }
    return ptrs[dev];
}


}  // namespace

extern "C" {

moe_options_t moe_default_options(void) {
    moe_options_t o;
    o.fast_math = 1;
    o.activation_clamp = NAN;
    o.debug_validate = 0;
    o.gemm_tiles = MOE_TILES_AUTO;
    return o;
}

size_t moe_workspace_bytes(const moe_shape_t* s) {
    if (!fused_shape_ok(s)) return 0;
    return make_layout(s).total;
}

size_t moe_dispatch_workspace_bytes(const moe_shape_t* s) {
    if (!shape_basic_ok(s) || s->H % 32) return 0;
    moe_shape_t t = *s;
    if (t.I % 32) t.I = 32;
    return make_layout(&t).routing_end;
}

int moe_workspace_views(const moe_shape_t* s, moe_workspace_views_t* v) {
    if (!v) return MOE_ERR_INVALID_ARG;
    if (!fused_shape_ok(s)) {
        memset(v, 0xFF, sizeof *v);
        return MOE_ERR_INVALID_ARG;
    }
    const Layout L = make_layout(s);
    v->counts = (int64_t)L.counts;
    v->offsets = (int64_t)L.offsets;
    v->pool_src = (int64_t)L.pool_src;
    v->slot_to_pool = (int64_t)L.slot_to_pool;
    v->pool_w = (int64_t)L.pool_w;
    v->pool_tok = (int64_t)L.pool_tok;
    v->x_q = (int64_t)L.x_q;
    v->x_s = (int64_t)L.tok_s;
    v->pool_s = (int64_t)L.pool_s;
    v->act_q = (int64_t)L.act_q;
    v->act_s = (int64_t)L.act_s;
    v->l2_out = (int64_t)L.l2_out;
    v->capacity_rows = L.cap;
    return MOE_OK;
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or unknown payload)";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or option for the gfx950 kernels";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_DEVICE: return "device is not gfx950 or a kernel launch failed";
        case MOE_ERR_BAD_ROUTING: return "an expert index was >= E";
        case MOE_ERR_TOO_LARGE:
            return "shape needs more workspace than the allocation-free entry's device scratch holds "
                   "(moe_workspace_bytes(s) > MOE_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

}  // extern "C"

namespace {

// The layer.  With `packed` set, the weight scales come from a buffer filled
// by moe_pack_weight_scales (S1, S2 unused); otherwise they are laid out
// into the workspace first.
int fused_forward(const moe_shape_t* s, const moe_options_t* opt, const void* x,
                  const int64_t* topk_idx, const float* topk_w, const uint8_t* W1q,
                  const uint8_t* S1, const uint8_t* W2q, const uint8_t* S2, const uint8_t* packed,
                  void* y, void* workspace, size_t workspace_bytes, moe_stream_t stream_,
                  bool b_tiled = false) {
    if (!shape_basic_ok(s)) return MOE_ERR_INVALID_ARG;
    const moe_options_t o = opt ? *opt : moe_default_options();
    if (!isnan(o.activation_clamp)) return MOE_ERR_UNSUPPORTED;
    if (o.gemm_tiles < MOE_TILES_AUTO || o.gemm_tiles > MOE_TILES_FUSED) return MOE_ERR_INVALID_ARG;
    if (!fused_shape_ok(s)) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    if (!x || !topk_idx || !topk_w || !W1q || !W2q || !y) return MOE_ERR_INVALID_ARG;
    if (packed) {
        if (reinterpret_cast<uintptr_t>(packed) % kAlign) return MOE_ERR_INVALID_ARG;
    } else {
        if (!S1 || !S2) return MOE_ERR_INVALID_ARG;
        if ((reinterpret_cast<uintptr_t>(S1) | reinterpret_cast<uintptr_t>(S2)) % 4)
            return MOE_ERR_INVALID_ARG;  // scale rows are read as 4-byte words
    }
    const Layout L = make_layout(s);
    if ((o.gemm_tiles == MOE_TILES_64 || o.gemm_tiles == MOE_TILES_128 || o.gemm_tiles == MOE_TILES_FUSED) &&
        !route_fused(L, s->E))
        return MOE_ERR_UNSUPPORTED;
    if (o.gemm_tiles == MOE_TILES_FUSED && s->I > kFusedMaxI) return MOE_ERR_UNSUPPORTED;
    if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) % kAlign))
        return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_DEVICE;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const int T = s->T, H = s->H, I = s->I, K = s->K;
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* pool_src = reinterpret_cast<int32_t*>(ws + L.pool_src);
    int32_t* slot_to_pool = reinterpret_cast<int32_t*>(ws + L.slot_to_pool);
    float* pool_w = reinterpret_cast<float*>(ws + L.pool_w);
    int32_t* pool_tok = reinterpret_cast<int32_t*>(ws + L.pool_tok);
    uint8_t* x_q = ws + L.x_q;
    uint8_t* pool_s = ws + L.pool_s;
    uint8_t* act_q = ws + L.act_q;
    uint8_t* act_s = ws + L.act_s;
    uint16_t* l2_out = reinterpret_cast<uint16_t*>(ws + L.l2_out);
    const uint8_t* s1t = packed ? packed : ws + L.s1t;
    const uint8_t* s2t = packed ? packed + align_up(packed_s1_bytes(s)) : ws + L.s2t;

    const int pc = prof_begin(stream);
    // weight scales into the packed k-major words the GEMMs load per K step
    // (unless the caller packed them once)
    if (!packed) launch_pack_scales(s, S1, S2, ws + L.s1t, ws + L.s2t, stream);
    prof_mark(pc, MOE_STAGE_WEIGHT_SCALES, stream);
    uint8_t* tok_s = ws + L.tok_s;
    // few rows per expert (e.g. a decode batch): the decode-shaped GEMMs over
    // the 64-row tile table that the routing writes.  With at most 1024
    // routed slots (routing inside the first launch) their L1 reads the
    // A-scale words by token instead of a pool copy, which saves a launch
    // (measured at 1024 slots with the tile-blocked weights: L1 +2.6 us, step
    // -2.9 us)
    const TilePlan plan = tile_plan(s, L, o.gemm_tiles);
    const bool decode = plan.rm == 1;
    const bool sa_by_token = decode && (int64_t)T * K <= kRouteSingleMax;
    const int drows = plan.rm ? dec_rows(plan.rm) : kDecRows;
    const int tpb = tokens_per_block(H);
    const int64_t nq = ((int64_t)T + tpb - 1) / tpb;
    int rc = MOE_OK;
    if ((int64_t)T * K <= kRouteSingleMax) {
        // one launch for a1-a4: the first blocks route the batch (256 slots
        // each, every one counting all slots itself) while the others
        // quantise the token rows
        const int64_t TKn = (int64_t)T * K;
        const int nroute = (int)((TKn + kRouteThreads - 1) / kRouteThreads);
        hipLaunchKernelGGL(k_quantise_route, dim3((unsigned)(nroute + nq)), dim3(256), route_lds_bytes(s->E),
                           stream, static_cast<const uint16_t*>(x), (int64_t)T, H, tpb, x_q, tok_s,
                           topk_idx, topk_w, TKn, s->E, bits_for(s->E), K, nroute, counts, offsets,
                           reinterpret_cast<MTile*>(ws + L.mtiles),
                           reinterpret_cast<int32_t*>(ws + L.num_mtiles),
                           reinterpret_cast<int32_t*>(ws + L.err_flag), pool_src, slot_to_pool, pool_w,
                           pool_tok, reinterpret_cast<MTile*>(ws + L.mtiles64),
                           reinterpret_cast<int32_t*>(ws + L.num_mtiles64), drows);
        prof_mark(pc, MOE_STAGE_DISPATCH, stream);
        prof_mark(pc, MOE_STAGE_ROUTE_SCAN, stream);
        prof_mark(pc, MOE_STAGE_ROUTE_SCATTER, stream);
        if (!sa_by_token)
            hipLaunchKernelGGL(k_pool_scales, dim3((unsigned)((L.cap + 255) / 256)), dim3(256), 0, stream,
                               reinterpret_cast<const uint32_t*>(tok_s), H / 128, pool_tok, offsets, s->E,
                               (int64_t)L.cap, reinterpret_cast<uint32_t*>(pool_s));
        prof_mark(pc, MOE_STAGE_POOL_SCALES, stream);
        rc = launch_status();
    } else {
        // every token row quantised once, token-major (the L1 GEMM gathers the
        // rows of its tiles through pool_tok); the a1 histogram in the same
        // launch
        const int ncount = route_blocks(L);
        hipLaunchKernelGGL(k_quantise_count, dim3((unsigned)(ncount + nq)), dim3(256),
                           sizeof(int32_t) * kRouteWaves * s->E, stream,
                           static_cast<const uint16_t*>(x), (int64_t)T, H, tpb, x_q, tok_s, topk_idx,
                           (int64_t)T * K, s->E, ncount, reinterpret_cast<int32_t*>(ws + L.seg_hist),
                           reinterpret_cast<int32_t*>(ws + L.seg_err),
                           route_fused(L, s->E) ? reinterpret_cast<int32_t*>(ws + L.blk_hist)
                                                : static_cast<int32_t*>(nullptr),
                           reinterpret_cast<int32_t*>(ws + L.blk_err));
        prof_mark(pc, MOE_STAGE_DISPATCH, stream);
        rc = run_routing(s, L, topk_idx, topk_w, ws, pool_tok, counts, offsets, pool_src, slot_to_pool,
                         pool_w, stream, true, pc, reinterpret_cast<const uint32_t*>(tok_s),
                         sa_by_token ? static_cast<uint32_t*>(nullptr) : reinterpret_cast<uint32_t*>(pool_s),
                         drows);
    }
    if (rc) return rc;
    if (o.debug_validate && (rc = check_routing_flag(ws, L, stream))) return rc;
    // an upper bound on the tiles of the second table (the grid's extra
    // workgroups find no tile and return)
    const int64_t TKn = (int64_t)T * K;
    const unsigned dec_grid_rows =
        (unsigned)(plan.rm ? TKn / dec_rows(plan.rm) + (s->E < TKn ? s->E : TKn) + 1 : 0);

    GemmArgs g1;
    memset(&g1, 0, sizeof g1);
    g1.A = x_q;
    g1.SA = pool_s;
    g1.B = W1q;
    g1.b_tiled = b_tiled ? 1 : 0;
    g1.SB = s1t;
    g1.sa_step = 4 * L.cap;
    g1.act_s_step = 4 * L.cap;
    g1.pool_tok = pool_tok;
    g1.T = T;
    g1.mtiles = reinterpret_cast<const MTile*>(ws + L.mtiles);
    g1.num_mtiles = reinterpret_cast<const int32_t*>(ws + L.num_mtiles);
    g1.Kdim = H;
    g1.N = 2 * I;
    g1.ntiles = I / 128;
    g1.pool_w = pool_w;
    g1.act_q = act_q;
    g1.act_s = act_s;
    g1.I = I;
    g1.fast_math = o.fast_math ? 1 : 0;
    if (plan.fused) {
        // both GEMMs in one launch, the activations kept in LDS
        g1.mtiles = reinterpret_cast<const MTile*>(ws + L.mtiles64);
        g1.num_mtiles = reinterpret_cast<const int32_t*>(ws + L.num_mtiles64);
        GemmArgs g2 = g1;
        g2.B = W2q;
        g2.SB = s2t;
        g2.Kdim = I;
        g2.N = H;
        g2.ntiles = H / kBN;
        g2.out = l2_out;
        hipLaunchKernelGGL(k_gemm_fused, dim3((dec_grid_rows + 7u) / 8u * 8u), dim3(kGemmThreads), 0, stream,
                           g1, g2);
    } else if (plan.l1) {
        if (sa_by_token) {
            g1.SA = tok_s;  // token-major words [T][H/128]
            g1.sa_step = 4;
            g1.sa_by_token = 1;
        }
        g1.mtiles = reinterpret_cast<const MTile*>(ws + L.mtiles64);
        g1.num_mtiles = reinterpret_cast<const int32_t*>(ws + L.num_mtiles64);
        hipLaunchKernelGGL(plan.rm == 1 ? (b_tiled ? k_gemm_l1_decode_nt : k_gemm_l1_decode) : k_gemm_l1_t128,
                           dim3(dec_grid_rows * (unsigned)g1.ntiles), dim3(kGemmThreads), 0, stream, g1);
    } else {
        hipLaunchKernelGGL(k_gemm_l1, dim3(gemm_grid(L.max_mtiles * g1.ntiles)), dim3(kGemmThreads), 0,
                           stream, g1);
    }
    prof_mark(pc, MOE_STAGE_GEMM_L1, stream);

    if (!plan.fused) {
        GemmArgs g2 = g1;
        g2.A = act_q;
        g2.SA = act_s;
        g2.sa_step = 4 * L.cap;  // packed k-major words of the pool rows
        g2.sa_by_token = 0;
        g2.pool_tok = nullptr;
        g2.B = W2q;
        g2.SB = s2t;
        g2.Kdim = I;
        g2.N = H;
        g2.ntiles = H / kBN;
        g2.out = l2_out;
        if (plan.l2) {
            g2.mtiles = reinterpret_cast<const MTile*>(ws + L.mtiles64);
            g2.num_mtiles = reinterpret_cast<const int32_t*>(ws + L.num_mtiles64);
            hipLaunchKernelGGL(plan.rm == 1 ? k_gemm_l2_decode : k_gemm_l2_t128,
                               dim3(dec_grid_rows * (unsigned)g2.ntiles), dim3(kGemmThreads), 0, stream, g2);
        } else {
            g2.mtiles = reinterpret_cast<const MTile*>(ws + L.mtiles);
            g2.num_mtiles = reinterpret_cast<const int32_t*>(ws + L.num_mtiles);
            hipLaunchKernelGGL(k_gemm_l2, dim3(gemm_grid(L.max_mtiles * g2.ntiles)), dim3(kGemmThreads), 0,
                               stream, g2);
        }
    }
    prof_mark(pc, MOE_STAGE_GEMM_L2, stream);

    {
        const int tpb = tokens_per_block(H), parts = combine_parts(T, H, tpb);
        hipLaunchKernelGGL(k_combine, dim3((unsigned)(((int64_t)T + tpb - 1) / tpb * parts)), dim3(256), 0,
                           stream, l2_out, slot_to_pool, static_cast<const float*>(nullptr), (int64_t)T, H,
                           K, tpb, parts, static_cast<uint16_t*>(y));
    }
    prof_mark(pc, MOE_STAGE_COMBINE, stream);
    return launch_status();
}

}  // namespace

extern "C" {

int moe_fused_forward(const moe_shape_t* s, const moe_options_t* opt, const void* x,
                      const int64_t* topk_idx, const float* topk_w, const uint8_t* W1q,
                      const uint8_t* S1, const uint8_t* W2q, const uint8_t* S2, void* y,
                      void* workspace, size_t workspace_bytes, moe_stream_t stream) {
    return fused_forward(s, opt, x, topk_idx, topk_w, W1q, S1, W2q, S2, nullptr, y, workspace,
                         workspace_bytes, stream);
}

size_t moe_packed_scales_bytes(const moe_shape_t* s) {
    if (!shape_basic_ok(s) || s->H % kBN || s->I % 128) return 0;  // T is not used here
    return packed_total_bytes(s);
}

int moe_pack_weight_scales(const moe_shape_t* s, const uint8_t* S1, const uint8_t* S2,
                           void* packed, size_t packed_bytes, moe_stream_t stream_) {
    if (!shape_basic_ok(s)) return MOE_ERR_INVALID_ARG;
    if (s->H % kBN || s->I % 128) return MOE_ERR_UNSUPPORTED;
    if (!S1 || !S2 || !packed) return MOE_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(S1) | reinterpret_cast<uintptr_t>(S2)) % 4 ||
        reinterpret_cast<uintptr_t>(packed) % kAlign)
        return MOE_ERR_INVALID_ARG;
    if (packed_bytes < packed_total_bytes(s)) return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_DEVICE;
    uint8_t* p = static_cast<uint8_t*>(packed);
    launch_pack_scales(s, S1, S2, p, p + align_up(packed_s1_bytes(s)),
                       reinterpret_cast<hipStream_t>(stream_));
    return launch_status();
}

int moe_fused_forward_packed(const moe_shape_t* s, const moe_options_t* opt, const void* x,
                             const int64_t* topk_idx, const float* topk_w, const uint8_t* W1q,
                             const uint8_t* W2q, const void* packed_scales, void* y,
                             void* workspace, size_t workspace_bytes, moe_stream_t stream) {
    if (!packed_scales) return MOE_ERR_INVALID_ARG;
    return fused_forward(s, opt, x, topk_idx, topk_w, W1q, nullptr, W2q, nullptr,
                         static_cast<const uint8_t*>(packed_scales), y, workspace,
                         workspace_bytes, stream);
}

size_t moe_packed_weights_bytes(const moe_shape_t* s) {
    if (!shape_basic_ok(s) || s->H % kBN || s->I % 128) return 0;
    return tiled_total_bytes(s);
}

int moe_pack_weights(const moe_shape_t* s, const uint8_t* W1q, const uint8_t* S1, const uint8_t* W2q,
                     const uint8_t* S2, void* packed, size_t packed_bytes, moe_stream_t stream_) {
    if (!shape_basic_ok(s)) return MOE_ERR_INVALID_ARG;
    if (s->H % kBN || s->I % 128) return MOE_ERR_UNSUPPORTED;
    if (!W1q || !W2q || !S1 || !S2 || !packed) return MOE_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(W1q) | reinterpret_cast<uintptr_t>(W2q)) % 16 ||
        (reinterpret_cast<uintptr_t>(S1) | reinterpret_cast<uintptr_t>(S2)) % 4 ||
        reinterpret_cast<uintptr_t>(packed) % kAlign)
        return MOE_ERR_INVALID_ARG;
    if (packed_bytes < tiled_total_bytes(s)) return MOE_ERR_WORKSPACE;
    if (!device_ok()) return MOE_ERR_DEVICE;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    uint8_t* p = static_cast<uint8_t*>(packed);
    const int H = s->H, I = s->I, E = s->E;
    const int64_t c1 = (int64_t)tiled_w1_bytes(s) / 16, c2 = (int64_t)tiled_w2_bytes(s) / 16;
    hipLaunchKernelGGL(k_pack_weights_tiled, dim3((unsigned)((c1 + 255) / 256)), dim3(256), 0, stream, W1q, p,
                       E, 2 * I, H, I, 1);
    hipLaunchKernelGGL(k_pack_weights_tiled, dim3((unsigned)((c2 + 255) / 256)), dim3(256), 0, stream, W2q,
                       p + tiled_w2_offset(s), E, H, I, I, 0);
    uint8_t* sc = p + tiled_scales_offset(s);
    launch_pack_scales(s, S1, S2, sc, sc + align_up(packed_s1_bytes(s)), stream);
    return launch_status();
}

int moe_fused_forward_prepacked(const moe_shape_t* s, const moe_options_t* opt, const void* x,
                                const int64_t* topk_idx, const float* topk_w, const void* packed_weights,
                                void* y, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
    if (!packed_weights) return MOE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(packed_weights) % kAlign) return MOE_ERR_INVALID_ARG;
    if (!shape_basic_ok(s)) return MOE_ERR_INVALID_ARG;
    const uint8_t* p = static_cast<const uint8_t*>(packed_weights);
    const bool sized = s->H % kBN == 0 && s->I % 128 == 0;  // else refused below, before any use
    return fused_forward(s, opt, x, topk_idx, topk_w, p, nullptr, sized ? p + tiled_w2_offset(s) : p, nullptr,
                         sized ? p + tiled_scales_offset(s) : p, y, workspace, workspace_bytes, stream, true);
}

int moe_fused_forward_packed_noalloc(const moe_shape_t* s, const moe_options_t* opt,
                                     const void* x, const int64_t* topk_idx, const float* topk_w,
                                     const uint8_t* W1q, const uint8_t* W2q,
                                     const void* packed_scales, void* y, moe_stream_t stream) {
    if (!packed_scales) return MOE_ERR_INVALID_ARG;
    // the limit is checked on the host, before anything touches the device
    if (shape_basic_ok(s) && fused_shape_ok(s) && s->T > 0 &&
        make_layout(s).total > kNoAllocScratchBytes)
        return MOE_ERR_TOO_LARGE;
    void* ws = nullptr;
    if (shape_basic_ok(s) && fused_shape_ok(s) && s->T > 0) {
        if (!device_ok()) return MOE_ERR_DEVICE;
        ws = scratch_device_ptr();
        if (!ws) return MOE_ERR_DEVICE;
    }
    return fused_forward(s, opt, x, topk_idx, topk_w, W1q, nullptr, W2q, nullptr,
                         static_cast<const uint8_t*>(packed_scales), y, ws,
                         ws ? kNoAllocScratchBytes : 0, stream);
}

int moe_dispatch(const moe_shape_t* s, const void* x, const int64_t* topk_idx, const float* topk_w,
                 int payload, int32_t* counts, int32_t* offsets, int32_t* pool_src,
                 int32_t* slot_to_pool, float* pool_w, void* pool, uint8_t* pool_scales,
                 void* workspace, size_t workspace_bytes, moe_stream_t stream_) {
    if (!shape_basic_ok(s)) return MOE_ERR_INVALID_ARG;
    if (payload != MOE_PAYLOAD_FP8_E4M3 && payload != MOE_PAYLOAD_BF16) return MOE_ERR_INVALID_ARG;
    if (s->H % 32) return MOE_ERR_UNSUPPORTED;
    if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
    moe_shape_t t = *s;
    if (t.I % 32) t.I = 32;
    const Layout L = make_layout(&t);
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    if (!workspace || workspace_bytes < L.routing_end ||
        (reinterpret_cast<uintptr_t>(workspace) % kAlign))
        return MOE_ERR_WORKSPACE;
    if (s->T == 0) {
        // nothing routed: one scan over zero segments writes counts = 0 and
        // offsets = 0
        if (!device_ok()) return MOE_ERR_DEVICE;
        uint8_t* ws = static_cast<uint8_t*>(workspace);
        const int scan_threads = 1024;
        hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(scan_threads), 0, stream,
                           reinterpret_cast<int32_t*>(ws + L.seg_hist),
                           reinterpret_cast<int32_t*>(ws + L.seg_err), 0, s->E,
                           reinterpret_cast<int32_t*>(ws + L.seg_base), counts, offsets,
                           reinterpret_cast<MTile*>(ws + L.mtiles),
                           reinterpret_cast<int32_t*>(ws + L.num_mtiles),
                           reinterpret_cast<int32_t*>(ws + L.err_flag));
        return launch_status();
    }
    if (!x || !topk_idx || !topk_w || !pool_src || !slot_to_pool || !pool_w || !pool ||
        (payload == MOE_PAYLOAD_FP8_E4M3 && !pool_scales))
        return MOE_ERR_INVALID_ARG;
    if (!device_ok()) return MOE_ERR_DEVICE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int rc = run_routing(s, L, topk_idx, topk_w, ws, nullptr, counts, offsets, pool_src, slot_to_pool,
                         pool_w, stream, false, -1, nullptr, nullptr);
    if (rc) return rc;
    const int tpb = tokens_per_block(s->H);
    if (payload == MOE_PAYLOAD_FP8_E4M3)
        hipLaunchKernelGGL(k_dispatch_fp8, dim3((unsigned)(((int64_t)s->T + tpb - 1) / tpb)),
                           dim3(256), 0, stream, static_cast<const uint16_t*>(x), (int64_t)s->T, s->H,
                           s->K, tpb, slot_to_pool,
                           static_cast<uint8_t*>(pool), pool_scales, static_cast<uint8_t*>(nullptr));
    else
        hipLaunchKernelGGL(k_dispatch_bf16, dim3(s->T), dim3(256), 0, stream,
                           static_cast<const uint16_t*>(x), s->H, s->K, slot_to_pool,
                           static_cast<uint16_t*>(pool));
    return launch_status();
}

int moe_combine(const moe_shape_t* s, const void* pool_out, const int32_t* slot_to_pool,
                const float* topk_w, void* y, moe_stream_t stream_) {
    if (!shape_basic_ok(s)) return MOE_ERR_INVALID_ARG;
    if (s->H % 8) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    if (!pool_out || !slot_to_pool || !y) return MOE_ERR_INVALID_ARG;
    if (!device_ok()) return MOE_ERR_DEVICE;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
    const int tpb = tokens_per_block(s->H), parts = combine_parts(s->T, s->H, tpb);
    hipLaunchKernelGGL(k_combine, dim3((unsigned)(((int64_t)s->T + tpb - 1) / tpb * parts)), dim3(256), 0,
                       stream, static_cast<const uint16_t*>(pool_out), slot_to_pool, topk_w,
                       (int64_t)s->T, s->H, s->K, tpb, parts, static_cast<uint16_t*>(y));
    return launch_status();
}

int moe_profile_start(int max_calls) {
    if (max_calls < 1 || max_calls > 4096) return MOE_ERR_INVALID_ARG;
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof = Profile();
    g_prof.ev.resize((size_t)max_calls * kMarks);
    // timing-only events: no system-scope fence (cache writeback and
    // invalidate) when one is recorded, which would otherwise open a gap of
    // several microseconds before every launch it separates
    for (auto& e : g_prof.ev)
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
            return MOE_ERR_DEVICE;
    g_prof.max_calls = max_calls;
    g_prof.on = true;
    return MOE_OK;
}

int moe_profile_stop(double* stage_ms, int* ncalls) {
    if (!g_prof.on || !stage_ms || !ncalls) return MOE_ERR_INVALID_ARG;
    int rc = MOE_OK;
    for (int k = 0; k < MOE_PROFILE_STAGES; ++k) stage_ms[k] = 0.0;
    // the events carry no fence, so wait for the device as a whole first
    if (hipDeviceSynchronize() != hipSuccess) rc = MOE_ERR_DEVICE;
    for (int c = 0; c < g_prof.ncalls && rc == MOE_OK; ++c) {
        if (hipEventSynchronize(g_prof.ev[c * kMarks + MOE_PROFILE_STAGES]) != hipSuccess) {
            rc = MOE_ERR_DEVICE;
            break;
        }
        for (int k = 0; k < MOE_PROFILE_STAGES; ++k) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, g_prof.ev[c * kMarks + k], g_prof.ev[c * kMarks + k + 1]) !=
                hipSuccess) {
                rc = MOE_ERR_DEVICE;
                break;
            }
            stage_ms[k] += ms;
        }
    }
    *ncalls = g_prof.ncalls;
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof = Profile();
    return rc;
}

const char* moe_profile_stage_name(int stage) {
    static const char* names[MOE_PROFILE_STAGES] = {"weight_scales", "dispatch",  "route_scan",
                                                    "route_scatter", "pool_scales", "gemm_l1",
                                                    "gemm_l2",       "combine"};
    return stage >= 0 && stage < MOE_PROFILE_STAGES ? names[stage] : "?";
}

}  // extern "C"
