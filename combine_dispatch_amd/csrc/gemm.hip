// gemm.hip -- grouped FP8 (e4m3) x FP4 (e2m1) block-scaled GEMMs for gfx950.
//
// a5/a8: for every expert e and every pool row r of that expert,
//   out[r][n] = sum_k deq(A[r][k]) * deq(B[e][n][k]),
// with one UE8M0 scale per 32 along k on both operands (page "DeepEP -> Mega
// MoE", "complete compute pipeline" snippet, the block-scaled MMA step;
// page "Normal vs Low-Latency", section 2, recipe (1,1,32)).
//   L1 epilogue (a6, a7): gate/up rounded to bf16, silu(gate) * up * w in
//   fp32, per-32-column amax, UE8M0 scale, e4m3 codes (page "DeepEP -> Mega
//   MoE", SwiGLU / amax / FP8 snippets; page "Dispatch/Combine in Mega MoE",
//   section 4.2 for the routing weight).
//   L2 epilogue: bf16 rows in pool order (same page, sections 4.2 and 5.1).
//
// MI355X design (not the pages' SM100 one):
//  - v_mfma_scale_f32_32x32x64_f8f6f4 with A = e4m3 (format 0), B = e2m1
//    (format 4), scales per lane; fp32 accumulators in AGPRs.
//  - 256 x 256 tile per 4-wave workgroup, each wave 64 rows x 256 columns
//    (2 x 8 MFMA tiles); K steps of 128 staged through three LDS stages by
//    direct global->LDS loads issued two steps ahead; 16-byte chunks XOR-swizzled so
//    that the 16 lanes of each ds_read_b128 phase hit distinct banks of the
//    64-bank LDS (A rows of 128 B: chunk ^ (row/2)%8; B rows of 64 B:
//    chunk ^ (row/4)%4).
//  - Expert-major m-tile table built on the device by the routing scan: no
//    host synchronisation.
//  - Persistent workgroups, one per CU; each XCD (own L2) works through a
//    contiguous run of tiles that share weights and activations.
//  - L1 tiles hold 128 gate and the matching 128 up columns, split so that
//    each wave has gate column j and up column j in the same lane and
//    register: the SwiGLU needs no data exchange.
//
// Operand lane layout of the 32x32x64 scaled MFMA (measured on gfx950):
//  A (e4m3, 8 VGPRs): lane l holds row l%32; bytes 0-15 are k = 16*(l/32)+0..15,
//    bytes 16-31 are k = 32 + 16*(l/32) + 0..15.
//  B (e2m1, 4 VGPRs): lane l holds column l%32, k = 32*(l/32) + 0..31, two per
//    byte, even k in the low nibble.
//  Scales: lane l gives the scale of row (column) l%32 for k-block l/32
//    (32 k each), in bits 0-7 of its scale register.
//  D (16 fp32): lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4,
//    column l%32.
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {

namespace {

constexpr int kL1 = 0;
constexpr int kL2 = 1;
// m-tiles per tile-order group.  Measured on the prefill workload (A/B on one
// machine): 1, 2 and 3 give the same L1 time and an L2 GEMM 1.5-2 % faster than
// 4; 8 is 3 % slower.
constexpr int kGroupM = 1;

// Which expert-matrix row (output column) holds LDS B row `nrow` of tile nt.
// LDS B row n is column c = n%32 of MFMA column tile j = n/32.  The order is
// chosen so that, after the MFMA, each lane holds adjacent output columns of a
// row:
//  L1: tiles 0-3 are gate, 4-7 the matching up columns; lane column c of tile
//      j is activation column 4c + j%4 of the tile's 128, so a lane holds 4
//      adjacent activation columns and the 8 lanes c = 8G..8G+7 hold the 32
//      columns of quantisation group G.
//  L2: lane column c of tile j is output column 8c + j of the tile's 256.
template <int MODE>
__device__ __forceinline__ int b_row(int nt, int nrow, int I) {
    const int j = nrow >> 5, c = nrow & 31;
    if (MODE == kL1) return (j < 4 ? 0 : I) + nt * 128 + 4 * c + (j & 3);
    return nt * kBN + 8 * c + j;
}

// The same for a narrow tile (at most 64 rows): every wave covers rows 0-63
// and multiplies two of the eight column tiles, chosen so that its outputs
// still fill whole quantisation groups (L1) or adjacent columns (L2):
//  L1: lane column c of tile j is activation column 32(j%4) + c (gate in
//      tiles 0-3, up in 4-7); wave w takes tiles w and w+4, i.e. gate and up
//      of quantisation group w, one column per lane.
//  L2: lane column c of tile j is output column 64(j/2) + 2c + j%2; wave w
//      takes tiles 2w and 2w+1, two adjacent output columns per lane.
// Row 0 of either order is the tile's first row, so the scalar bases agree.
template <int MODE>
__device__ __forceinline__ int b_row_narrow(int nt, int nrow, int I) {
    const int j = nrow >> 5, c = nrow & 31;
    if (MODE == kL1) return (j < 4 ? 0 : I) + nt * 128 + 32 * (j & 3) + c;
    return nt * kBN + 64 * (j >> 1) + 2 * c + (j & 1);
}
// Tiles with at most this many rows run narrow.
constexpr int kNarrowRows = 64;

// Per-lane offsets of a wave's eight A loads and its A-scale load (named
// fields, so that they stay in registers: an array indexed through the load
// helpers ends up in scratch memory).
struct LoadOffs {
    uint32_t a0, a1, a2, a3, a4, a5, a6, a7, sa;
    __device__ __forceinline__ uint32_t a(int p) const {
        return p == 0 ? a0 : p == 1 ? a1 : p == 2 ? a2 : p == 3 ? a3 : p == 4 ? a4 : p == 5 ? a5
             : p == 6 ? a6 : a7;
    }
    __device__ __forceinline__ void set_a(int p, uint32_t v) {
        if (p == 0) a0 = v; else if (p == 1) a1 = v; else if (p == 2) a2 = v; else if (p == 3) a3 = v;
        else if (p == 4) a4 = v; else if (p == 5) a5 = v; else if (p == 6) a6 = v; else a7 = v;
    }
};

// MFMA operands of one 64-wide K sub-step for one wave: A fragments of its 2
// row tiles, B fragments of the 8 column tiles.
struct SubFrags {
    v8i a[2];
    v4i b[8];
};

// Scale words of one K step for one wave: the word of each of its 2 A row
// tiles and 8 B column tiles (lane row / column l%32).  Words hold the bytes
// of k-blocks (0, 2, 1, 3) of the step; shifted right by 16 in lanes 32-63
// they hold k-block 2s + l/32 in byte s, so sub-step s selects byte s.
struct ScaleWords {
    int a[2];
    int b[8];
};

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS byte address of a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// Direct global -> LDS loads (global_load_lds_dwordx4 / _dword): lane l's
// data lands at LDS address m0 + 16 l (4 l).  Written as inline asm so that
// the compiler neither reorders LDS reads around them nor inserts its own
// conservative vmcnt waits; the main loop counts them itself.  M0 is set
// here.  The compiler treats M0 as a reserved register (a clobber of it is
// ignored), so nothing else may use M0 in these kernels: a test over the
// assembly of the build checks that every instruction reading M0 follows
// one of these moves directly.
// The asm operands must sit in SGPRs; the values are wave-uniform by
// construction and readfirstlane states that to the compiler (free when it
// already knows).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma_x4(uint32_t lds, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory");
}
__device__ __forceinline__ void dma_x1(uint32_t lds, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory");
}
// The same with the non-temporal hint, for operands that are streamed once
// (a plain read stream reaches 7.2 TB/s with it, 6.3 TB/s without, on one
// MI355X).
__device__ __forceinline__ void dma_x4_nt(uint32_t lds, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory");
}
__device__ __forceinline__ void dma_x1_nt(uint32_t lds, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2 nt"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(uniform_ptr(sbase))
                 : "memory");
}
// Wait for this wave's direct loads except the newest 14, 21 or 22 (or all), then a
// workgroup barrier.  No memory fence: the data already sits in LDS.
__device__ __forceinline__ void barrier_after_vmcnt14() {
    asm volatile("s_waitcnt vmcnt(14) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_after_vmcnt21() {
    asm volatile("s_waitcnt vmcnt(21) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_after_vmcnt22() {
    asm volatile("s_waitcnt vmcnt(22) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void barrier_after_vmcnt0() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Every wave's LDS reads are done (the stages may be overwritten).
__device__ __forceinline__ void lds_reads_done_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// All of this wave's direct loads have landed (none may still write LDS when
// the workgroup ends).
__device__ __forceinline__ void wait_all_loads() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// Buffer resource over [base, base + bytes): raw buffer stores at offsets at or
// past `bytes` are dropped by the hardware range check (third descriptor word
// of a raw untyped gfx9 buffer).  The epilogues use it to skip the rows past
// the end of a short tile without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Cache policy of the epilogue stores: non-temporal (the gfx940-family NT
// bit) in the persistent GEMMs.  Their outputs are read back only by the next
// kernel, long after they have left the caches, so they should not push out
// the operand tiles that the XCD's workgroups share through its L2.  The
// decode-shaped GEMMs store with the default policy: their outputs are small
// and the next kernel reads them within microseconds (measured about 1 us
// faster per layer at 128 tokens, no difference with the NT bit on prefill).
constexpr int kStoreNT = 2;
constexpr int kStoreDecode = 0;

// A copy of v that the compiler cannot compute before this point: keeps the
// epilogue's per-lane address arithmetic (the same for every tile) from being
// hoisted out of the tile loop, where it would hold registers across the K
// loop.
__device__ __forceinline__ int late_copy(int v) {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(v));
    return r;
}

// One LDS stage: A tile [256 rows][128 B], B tile [256 rows][64 B], then one
// kilobyte of A scale words and one of B scale words.
//
// Persistent: one workgroup per CU loops over tiles.  The grid is a multiple
// of 8 and the hardware places workgroup b on XCD b % 8; XCD x owns the
// logical tiles [total*x/8, total*(x+1)/8) and its workgroups take them
// round-robin, so the ~32 workgroups of an XCD work on consecutive tiles of
// one group and share operands through that XCD's L2.  The stream of K
// steps runs on across tiles: the last three steps of a tile issue the first
// loads of the next one at the steady rate, so they land while the epilogue
// runs.  (The host sizes the grid so that no workgroup has more than
// kTileCache tiles.)
template <int MODE>
__device__ __forceinline__ void gemm_persistent(const GemmArgs& g, uint8_t* st0, uint8_t* st1,
                                                uint8_t* st2, float* s_wa, float* s_wb,
                                                MTile* s_tiles, int32_t* s_tok) {
    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int lane = tid & 63;
    const int wm = wid;  // rows 64*wm .. 64*wm+63 of the tile, all 256 columns
    const int h = lane >> 5, l32 = lane & 31;

    const int Kdim = g.Kdim;
    const int nk = Kdim / kBK;

    // Tile order: groups of kGroupM m-tiles x all n-tiles, m fastest; with
    // one m-tile per group the ~32 workgroups of an XCD cover all n-tiles of
    // one or two m-tiles at a time (sharing those A rows through its L2)
    // while the expert's B n-tiles come round again for the next m-tile.
    const int num_m = *g.num_mtiles;
    const int total = num_m * g.ntiles;
    const int xcd = blockIdx.x & 7, nj = (int)gridDim.x >> 3;
    const int t_hi = (int)((int64_t)total * (xcd + 1) / 8);
    int logical = (int)((int64_t)total * xcd / 8) + (int)(blockIdx.x >> 3);
    if (logical >= t_hi) return;
    // This workgroup's tiles, in order: the first kTileCache records
    // {expert, row0, nrows, n-tile} are gathered into LDS once, so moving to
    // the next tile costs an LDS read instead of a dependent global load.
    auto record = [&](int lg) __attribute__((always_inline)) {
        const int group = lg / (kGroupM * g.ntiles);
        const int in_group = lg - group * (kGroupM * g.ntiles);
        const int gm = min(kGroupM, num_m - group * kGroupM);
        MTile t = g.mtiles[group * kGroupM + in_group % gm];
        t.pad = in_group / gm;
        return t;
    };
    {
        const int mine = (t_hi - logical + nj - 1) / nj;
        for (int i = tid; i < min(mine, kTileCache); i += kGemmThreads) s_tiles[i] = record(logical + i * nj);
        __syncthreads();
    }
    int e = 0, row0 = 0, nrows = 0, nt = 0, tile_i = 0;
    auto take = [&](const MTile& t) __attribute__((always_inline)) {
        e = __builtin_amdgcn_readfirstlane(t.expert);
        row0 = __builtin_amdgcn_readfirstlane(t.row0);
        nrows = __builtin_amdgcn_readfirstlane(t.nrows);
        nt = __builtin_amdgcn_readfirstlane(t.pad);
    };
    take(s_tiles[0]);

    // ---- global -> LDS direct loads --------------------------------------
    // global_load_lds_dwordx4 writes lane l's 16 bytes to LDS at M0 + 16 l,
    // so one wave instruction fills 1 KiB of LDS; the lane's global address
    // chooses which chunk lands there.  Addresses are a wave-uniform SGPR base
    // (advanced by k each step) plus a per-lane 32-bit offset.
    //
    // A: 2048 16-byte chunks per step.  Chunk q = tid + 256 i (i = 0..7) is LDS
    // row q/8, physical chunk q%8, holding logical chunk (q%8) ^ ((row/2)%8).
    const int a_chunk = (tid & 7) ^ ((tid >> 4) & 7);
    const uint32_t a_off = (uint32_t)((tid >> 3) * Kdim + 16 * a_chunk);
    // B: 1024 chunks; chunk q = tid + 256 i is LDS row q/4 (B row b_row(q/4)),
    // physical chunk q%4, logical chunk (q%4) ^ ((row/4)%4).
    const int b_chunk = (tid & 3) ^ ((tid >> 4) & 3);
    const int b_ld = Kdim / 2;
    // the B codes' row stride, bytes per K step and the I of the row order
    // (tile-blocked: rows of a block 64 bytes apart, blocks of a tile
    // consecutive, L1's up rows right after its 128 gate rows)
    const int b_rs = g.b_tiled ? kBK / 2 : b_ld;
    const int64_t b_ks = g.b_tiled ? (int64_t)kBTileBytes : kBK / 2;
    const int bI = g.b_tiled ? 128 : g.I;
    // Load q (0..3) covers LDS B rows 64q + tid/4; with the column order of
    // b_row its expert rows differ from those of load 0 by a wave-uniform
    // number of rows, which goes into the scalar base.
    // (row offsets relative to the tile's first B row do not depend on the tile)
    const uint32_t b_off = (uint32_t)((b_row<MODE>(0, (tid >> 2), bI) - b_row<MODE>(0, 0, bI)) * b_rs + 16 * b_chunk);
    // per-load lane offsets (in vector registers: the scalar registers hold
    // one base per operand, advanced by K each step)
    // (L1 gathers its A rows from token rows: there the offsets change per
    // tile, see gather_offsets)
    LoadOffs lo;
#pragma unroll
    for (int p = 0; p < 8; ++p) lo.set_a(p, a_off + 32 * p * Kdim);
    const uint32_t b_off0 = b_off,
                   b_off1 = b_off + (b_row<MODE>(0, 64, bI) - b_row<MODE>(0, 0, bI)) * b_rs,
                   b_off2 = b_off + (b_row<MODE>(0, 128, bI) - b_row<MODE>(0, 0, bI)) * b_rs,
                   b_off3 = b_off + (b_row<MODE>(0, 192, bI) - b_row<MODE>(0, 0, bI)) * b_rs;
    // scales: packed k-major words, one 4-byte word (4 k-blocks) per row per
    // step, the words of a step contiguous over rows.  LDS word p of the A
    // scales is row tile p%2 of wave p/64, lane row (p%64)/2, so a lane's two
    // words are adjacent; LDS word p of the B scales is column tile p%8,
    // lane column p/8, so a lane's eight words are adjacent.  Thread tid loads
    // LDS word tid of each, so it picks its source row accordingly.
    const int64_t sa_step = g.sa_step;
    const int sa_row = (tid & ~63) + 32 * (tid & 1) + ((tid & 63) >> 1);
    lo.sa = (uint32_t)(4 * sa_row);
    const int64_t sb_step = (int64_t)g.N * 4;
    const uint32_t sb_off = (uint32_t)((b_row<MODE>(0, 32 * (tid & 7) + (tid >> 3), g.I) - b_row<MODE>(0, 0, g.I)) * 4);
    // the same lane offsets for the column order of narrow tiles
    const uint32_t nb_off = (uint32_t)((b_row_narrow<MODE>(0, (tid >> 2), bI) - b_row_narrow<MODE>(0, 0, bI)) * b_rs + 16 * b_chunk);
    const uint32_t nb_off0 = nb_off,
                   nb_off1 = nb_off + (b_row_narrow<MODE>(0, 64, bI) - b_row_narrow<MODE>(0, 0, bI)) * b_rs,
                   nb_off2 = nb_off + (b_row_narrow<MODE>(0, 128, bI) - b_row_narrow<MODE>(0, 0, bI)) * b_rs,
                   nb_off3 = nb_off + (b_row_narrow<MODE>(0, 192, bI) - b_row_narrow<MODE>(0, 0, bI)) * b_rs;
    const uint32_t nsb_off = (uint32_t)((b_row_narrow<MODE>(0, 32 * (tid & 7) + (tid >> 3), g.I) - b_row_narrow<MODE>(0, 0, g.I)) * 4);
    // column order of the tile whose loads go out when NAR below is 2: 1 for
    // a narrow tile (wave-uniform)
    int lnar = 0;
    // scalar bases of the current tile
    const uint8_t *a_base, *b_base, *sa_base, *sb_base;
    auto set_bases = [&]() __attribute__((always_inline)) {
        const int b_r0 = b_row<MODE>(nt, 0, g.I);
        a_base = MODE == kL1 ? g.A : g.A + (int64_t)row0 * Kdim;
        b_base = g.b_tiled ? g.B + ((int64_t)e * g.ntiles + nt) * (int64_t)nk * kBTileBytes
                           : g.B + ((int64_t)e * g.N + b_r0) * b_ld;
        sa_base = g.SA + (int64_t)row0 * 4;
        sb_base = g.SB + (int64_t)e * (Kdim / 128) * sb_step + (int64_t)b_r0 * 4;
    };
    set_bases();
    // L1: pool row r of a tile reads A row pool_tok[row0 + r] (the
    // token-major quantised input), so the per-load lane offsets follow the
    // tile: load p covers tile rows 32p + tid/8.  (The A-scale words are
    // gathered into pool order beforehand: read scattered, 4 bytes a row,
    // they would cost as much L2 traffic as the codes.)  Token indices are
    // clamped to T-1, so rows past the routed ones (whose entries hold
    // anything) still read inside the buffer.  The offsets are 32-bit: the
    // host checks T * Kdim < 2^32.
    const uint32_t tmax = (uint32_t)(g.T - 1);
    auto gather_offsets = [&](auto tok_at, LoadOffs& o) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 8; ++p)
            o.set_a(p, min((uint32_t)tok_at((tid >> 3) + 32 * p), tmax) * (uint32_t)Kdim + 16u * (uint32_t)a_chunk);
    };
    LoadOffs nlo = lo;  // the next tile's (L1)
    if constexpr (MODE == kL1) {
        const int32_t* tk = g.pool_tok + row0;
        gather_offsets([&](int r) { return tk[r]; }, lo);
        // consume them here: the compiler's wait for these loads then lands
        // before the pipeline starts, not at their first use inside the K
        // loop (where it would also wait for the direct loads in flight)
        asm volatile("" ::"v"(lo.a0), "v"(lo.a1), "v"(lo.a2), "v"(lo.a3), "v"(lo.a4), "v"(lo.a5),
                     "v"(lo.a6), "v"(lo.a7));
    }
    // LDS stages of the current step k, of k+1 and of k+2; the rotation runs
    // on across tiles.
    const uint8_t* cur = st0;
    const uint8_t* next = st1;
    const uint8_t* third = st2;
    const uint32_t w_dst16 = (uint32_t)(64 * wid * 16);
    const uint32_t w_dst4 = (uint32_t)(64 * wid * 4);

    // 14 loads per wave per step (8 A, 4 B, 2 scale dwords), load number
    // 0..13.  A step's loads go out in two halves of 7, spread one per two
    // MFMAs: first half-loads h = 0, second h = 1.
    // NAR: 0 a full tile; 1 a narrow tile, whose A rows past 63 are not
    // needed (a 4-byte stand-in load keeps the count of loads per step); 2
    // the column order chosen by lnar, all A rows loaded.
    auto issue_piece = [&](uint32_t st, int kk, int p, auto nar) __attribute__((always_inline)) {
        constexpr int NAR = decltype(nar)::value;
        const int k0 = kk * kBK;
        if (p < 8) {
            if (NAR == 1 && p >= 2)
                dma_x1(st + w_dst16 + 4096 * p, a_base + k0, lo.a0);
            else
                dma_x4(st + w_dst16 + 4096 * p, a_base + k0, lo.a(p));
        } else if (p < 12) {
            const uint32_t fo = p == 8 ? b_off0 : p == 9 ? b_off1 : p == 10 ? b_off2 : b_off3;
            const uint32_t no = p == 8 ? nb_off0 : p == 9 ? nb_off1 : p == 10 ? nb_off2 : nb_off3;
            const uint32_t off = NAR == 0 ? fo : NAR == 1 ? no : (lnar ? no : fo);
            dma_x4(st + kStageA + w_dst16 + 4096 * (p - 8), b_base + kk * b_ks, off);
        } else if (p == 12) {
            dma_x1(st + kStageA + kStageB + w_dst4, sa_base + kk * sa_step, lo.sa);
        } else if (p == 13) {
            const uint32_t off = NAR == 0 ? sb_off : NAR == 1 ? nsb_off : (lnar ? nsb_off : sb_off);
            dma_x1(st + kStageA + kStageB + kStageSA + w_dst4, sb_base + kk * sb_step, off);
        }
    };
    // Load of half `hf` that goes beside MFMA number g (0..15) of a sub-step.
    auto issue_spread = [&](uint32_t st, int kk, int hf, int g, auto nar) __attribute__((always_inline)) {
        if ((g & 1) == 0 && g < 14) issue_piece(st, kk, 7 * hf + (g >> 1), nar);
    };
    auto issue_half = [&](uint32_t st, int kk, int hf, auto nar) __attribute__((always_inline)) {
#pragma unroll
        for (int p = 0; p < 7; ++p) issue_piece(st, kk, 7 * hf + p, nar);
    };
    const std::integral_constant<int, 0> nar_full;
    const std::integral_constant<int, 1> nar_narrow;
    const std::integral_constant<int, 2> nar_sel;

    v16f acc[2][8];

    // ---- fragment reads --------------------------------------------------
    // A row of row-tile i: 64*wm + 32*i + l32, so (row/2)%8 == (l32/2)%8.
    const int a_frag_row = 64 * wm + l32;
    const int a_sw = (l32 >> 1) & 7;
    // B row of column tile j: 32*j + l32, so (row/4)%4 == (l32/4)%4.
    const int b_sw = (l32 >> 2) & 3;

    // Operand reads of sub-step s (0 or 1) of the step held in an LDS stage,
    // split into the pieces read next to each MFMA, in the order the next
    // sub-step's MFMAs (row tile 0 with column tiles 0..7, then row tile 1)
    // consume them: row tile 0, the column tiles, row tile 1.
    // ACT (0..2): how many of the wave's two row tiles hold rows of the tile
    // (a short last tile of an expert leaves some waves with none); reads and
    // MFMAs of the other row tiles are skipped.
    auto read_piece = [&](SubFrags& f, const uint8_t* base, int s, int g, auto act) __attribute__((always_inline)) {
        constexpr int ACT = decltype(act)::value;
        if (ACT == 0) return;
        const uint8_t* sA = base;
        const uint8_t* sB = base + kStageA;
        auto read_a = [&](int i, int part) __attribute__((always_inline)) {
            const uint8_t* rowp = sA + (a_frag_row + 32 * i) * kBK;
            const uint4 v = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * s + 2 * part + h) ^ a_sw));
            if (part == 0) {
                f.a[i][0] = (int)v.x; f.a[i][1] = (int)v.y; f.a[i][2] = (int)v.z; f.a[i][3] = (int)v.w;
            } else {
                f.a[i][4] = (int)v.x; f.a[i][5] = (int)v.y; f.a[i][6] = (int)v.z; f.a[i][7] = (int)v.w;
            }
        };
        if (g < 2) {
            read_a(0, g);
        } else if (g < 10) {
            const int j = g - 2;
            const uint8_t* rowp = sB + (32 * j + l32) * (kBK / 2);
            const uint4 v = *reinterpret_cast<const uint4*>(rowp + 16 * ((2 * s + h) ^ b_sw));
            f.b[j] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        } else if (g < 12) {
            if (ACT > 1) read_a(1, g - 10);
        }
    };
    // Scale words of a step: part 0 the two A words (8 bytes), parts 1 and 2
    // the B words 0-3 and 4-7 (16 bytes each).
    auto read_scales = [&](ScaleWords& w, const uint8_t* base, int part) __attribute__((always_inline)) {
        const uint8_t* sSA = base + kStageA + kStageB;
        const uint8_t* sSB = sSA + kStageSA;
        if (part == 0) {
            const uint2 v = *reinterpret_cast<const uint2*>(sSA + 256 * wm + 8 * l32);
            w.a[0] = (int)v.x; w.a[1] = (int)v.y;
        } else {
            const uint4 v = *reinterpret_cast<const uint4*>(sSB + 32 * l32 + 16 * (part - 1));
            const int j0 = 4 * (part - 1);
            w.b[j0] = (int)v.x; w.b[j0 + 1] = (int)v.y; w.b[j0 + 2] = (int)v.z; w.b[j0 + 3] = (int)v.w;
        }
    };
    auto read_all = [&](SubFrags& f, ScaleWords& w, const uint8_t* base, int s, auto act) __attribute__((always_inline)) {
        if (decltype(act)::value == 0) return;
#pragma unroll
        for (int g = 0; g < 12; ++g) read_piece(f, base, s, g, act);
#pragma unroll
        for (int part = 0; part < 3; ++part) read_scales(w, base, part);
    };
    // Scale words read beside the pieces of the next step's sub-step 0.
    auto read_piece_and_scales = [&](SubFrags& f, ScaleWords& w, const uint8_t* base, int g, auto act) __attribute__((always_inline)) {
        if (decltype(act)::value == 0) return;
        read_piece(f, base, 0, g, act);
        if (g == 0) read_scales(w, base, 0);
        if (g == 1) read_scales(w, base, 1);
        if (g == 5) read_scales(w, base, 2);
    };
    // Words as read -> words the MFMAs use (see ScaleWords); done beside the
    // first MFMA that needs each.
    const int hs = 16 * h;
    auto shift_for = [&](ScaleWords& c, const ScaleWords& n, int g, auto act) __attribute__((always_inline)) {
        if (decltype(act)::value == 0) return;
        if (g == 0) { c.a[0] = (int)((uint32_t)n.a[0] >> hs); c.b[0] = (int)((uint32_t)n.b[0] >> hs); }
        if (g > 0 && g < 8) c.b[g] = (int)((uint32_t)n.b[g] >> hs);
        if (g == 8) c.a[1] = (int)((uint32_t)n.a[1] >> hs);
    };
    // MFMA number g (0..15) of sub-step S: row tile g/8, column tile g%8;
    // scale byte S of the words.
    auto mfma_one = [&](const SubFrags& f, const ScaleWords& w, auto sub, int g, auto act) __attribute__((always_inline)) {
        constexpr int S = decltype(sub)::value;
        const int i = g >> 3, j = g & 7;
        if (i >= decltype(act)::value) return;
        const v8i b = v8i{f.b[j][0], f.b[j][1], f.b[j][2], f.b[j][3], 0, 0, 0, 0};
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], b, acc[i][j], 0, 4, S,
                                                                     w.a[i], S, w.b[j]);
    };
    const std::integral_constant<int, 0> sub0;
    const std::integral_constant<int, 1> sub1;

    // ---- narrow tiles ------------------------------------------------------
    // Wave wid's two column tiles (see b_row_narrow); its B fragments and B
    // scale words sit in slots 0 and 1 of SubFrags::b and ScaleWords::b, its
    // accumulators in acc[i][0] and acc[i][1].
    const int jn0 = MODE == kL1 ? wid : 2 * wid;
    const int jn1 = MODE == kL1 ? wid + 4 : 2 * wid + 1;
    // Reads of sub-step s, in the order the MFMAs use them: row tile 0 (two
    // 16-byte pieces), column tiles jn0 and jn1, row tile 1 (two pieces).
    auto read_piece_n = [&](SubFrags& f, const uint8_t* base, int s, int p) __attribute__((always_inline)) {
        const uint8_t* sA = base;
        const uint8_t* sB = base + kStageA;
        auto read_a = [&](int i, int part) __attribute__((always_inline)) {
            const uint8_t* rowp = sA + (l32 + 32 * i) * kBK;
            const uint4 v = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * s + 2 * part + h) ^ a_sw));
            if (part == 0) {
                f.a[i][0] = (int)v.x; f.a[i][1] = (int)v.y; f.a[i][2] = (int)v.z; f.a[i][3] = (int)v.w;
            } else {
                f.a[i][4] = (int)v.x; f.a[i][5] = (int)v.y; f.a[i][6] = (int)v.z; f.a[i][7] = (int)v.w;
            }
        };
        if (p < 2) {
            read_a(0, p);
        } else if (p < 4) {
            const uint8_t* rowp = sB + (32 * (p == 2 ? jn0 : jn1) + l32) * (kBK / 2);
            const uint4 v = *reinterpret_cast<const uint4*>(rowp + 16 * ((2 * s + h) ^ b_sw));
            f.b[p - 2] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        } else {
            read_a(1, p - 4);
        }
    };
    // Scale words of a step: the two A words of rows 0-63 and the B words of
    // column tiles jn0 and jn1 (LDS word 8c + j is column tile j, lane column c).
    auto read_scales_n = [&](ScaleWords& w, const uint8_t* base) __attribute__((always_inline)) {
        const uint8_t* sSA = base + kStageA + kStageB;
        const uint8_t* sSB = sSA + kStageSA;
        const uint2 v = *reinterpret_cast<const uint2*>(sSA + 8 * l32);
        w.a[0] = (int)v.x;
        w.a[1] = (int)v.y;
        w.b[0] = *reinterpret_cast<const int*>(sSB + 4 * (8 * l32 + jn0));
        w.b[1] = *reinterpret_cast<const int*>(sSB + 4 * (8 * l32 + jn1));
    };
    auto shift_n = [&](ScaleWords& c, const ScaleWords& n) __attribute__((always_inline)) {
        c.a[0] = (int)((uint32_t)n.a[0] >> hs);
        c.a[1] = (int)((uint32_t)n.a[1] >> hs);
        c.b[0] = (int)((uint32_t)n.b[0] >> hs);
        c.b[1] = (int)((uint32_t)n.b[1] >> hs);
    };
    // MFMA q (0..3) of sub-step S: row tile q/2, column slot q%2.
    auto mfma_n = [&](const SubFrags& f, const ScaleWords& w, auto sub, int q) __attribute__((always_inline)) {
        constexpr int S = decltype(sub)::value;
        const int i = q >> 1, jj = q & 1;
        const v8i b = v8i{f.b[jj][0], f.b[jj][1], f.b[jj][2], f.b[jj][3], 0, 0, 0, 0};
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], b, acc[i][jj], 0, 4, S,
                                                                      w.a[i], S, w.b[jj]);
    };

    // The epilogue of a finished tile (its row0, nrows, nt and routing weights).
    auto epilogue = [&](const int row0, const int nrows, const int nt, const float* s_w) __attribute__((always_inline)) {
    // ---- epilogue ------------------------------------------------------------
        const int lane = late_copy(tid & 63);
        const int h = lane >> 5, l32 = lane & 31;
    // Register r of tile (i, j) is row 64*wm + 32*i + 8*(r/4) + 4*h + r%4;
    // thanks to the column order of the B rows each lane holds adjacent output
    // columns of that row, so rows go straight to global memory: 32 lanes
    // store one contiguous run of the row (no LDS, no lane exchanges).
    // Stores go through buffer resources that end at the tile's last row, so
    // rows past the end of a short tile are dropped without branches; a row
    // tile with no rows at all is skipped (a wave-uniform test).
    if (MODE == kL2) {
        const int N = g.N;
        uint8_t* out_base = reinterpret_cast<uint8_t*>(g.out + (int64_t)row0 * N + nt * kBN);  // wave-uniform
        const __amdgpu_buffer_rsrc_t out_rs = rows_rsrc(out_base, nrows * N * 2);
        // byte offset of row 64*wm + 4*h, columns 8*l32..: each row register
        // adds a wave-uniform multiple of the row pitch
        const int lane_off = 2 * ((64 * wm + 4 * h) * N + 8 * l32);
        const int pitch = 2 * N;
        auto rows = [&](auto partial) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (decltype(partial)::value && 64 * wm + 32 * i >= nrows) continue;  // no rows
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // columns 8*l32 + j, j = 0..7: 16 bytes
                    float c[8];  // read from the accumulator registers where used
#pragma unroll
                    for (int j = 0; j < 8; ++j) asm("v_accvgpr_read_b32 %0, %1" : "=v"(c[j]) : "a"(acc[i][j][r]));
                    const u32x4 v = {pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3]),
                                     pack_bf16x2(c[4], c[5]), pack_bf16x2(c[6], c[7])};
                    const int step = 32 * i + 8 * (r >> 2) + (r & 3);
                    __builtin_amdgcn_raw_buffer_store_b128(v, out_rs, lane_off + pitch * step, 0, kStoreNT);
                }
            }
        };
        rows(std::true_type{});
    } else {
        // Activation columns 4*l32 + jj (jj = 0..3) of the tile's 128: gate in
        // tile jj, up in tile jj + 4.  Quantisation group G = l32/8 spans the
        // 8 lanes l32 = 8G..8G+7, so the group amax is a max over 4 registers
        // and then over 8 lanes (three DPP steps inside the lane's row).
        // Rows go in blocks of 4 consecutive rows (registers r = 4*rq + 0..3),
        // computed without branches so the four rows interleave; then each
        // row's 4 code bytes are one dword store, and lanes l32 = 8G + rr
        // (rr < 4) store the scale byte of row rr, group G: one byte store per
        // block writes the block's 16 contiguous scale bytes.
        const int I = g.I;
        uint8_t* q_base = g.act_q + (int64_t)row0 * I + nt * 128;                 // wave-uniform
        uint8_t* s_base = g.act_s + (int64_t)nt * g.act_s_step + (int64_t)row0 * 4;  // wave-uniform
        const __amdgpu_buffer_rsrc_t q_rs = rows_rsrc(q_base, nrows * I);
        const __amdgpu_buffer_rsrc_t s_rs = rows_rsrc(s_base, nrows * 4);
        const int rsel = l32 & 7;
        const uint32_t bshift = 8u * (uint32_t)(rsel & 3);
        const int q_lane = (64 * wm + 4 * h) * I + 4 * l32;  // row 64*wm + 4*h, this lane's 4 codes
        const int G = l32 >> 3, gbyte = ((G & 1) << 1) | (G >> 1);
        auto rows = [&](auto fast, auto partial) __attribute__((always_inline)) {
            constexpr bool kPartial = decltype(partial)::value;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (kPartial && 64 * wm + 32 * i >= nrows) continue;  // no rows
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int lrow0 = 64 * wm + 32 * i + 8 * rq + 4 * h;
                    const float4 w4 = *reinterpret_cast<const float4*>(s_w + lrow0);
                    const float wr[4] = {w4.x, w4.y, w4.z, w4.w};
                    // In phases over the block's 16 elements (reads and bf16
                    // rounding, exp, reciprocal, products), so that 16
                    // independent chains hide the latency of the
                    // transcendentals.
                    float gt[4][4], up[4][4], a[4][4];
                    uint32_t m[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            // gate and up rounded to bf16 by one conversion,
                            // read from the accumulator registers where used
                            // (else the compiler copies all 256 up front)
                            const int r = 4 * rq + rr;
                            float ga, ua;
                            asm("v_accvgpr_read_b32 %0, %1" : "=v"(ga) : "a"(acc[i][jj][r]));
                            asm("v_accvgpr_read_b32 %0, %1" : "=v"(ua) : "a"(acc[i][jj + 4][r]));
                            const uint32_t gu = pack_bf16x2(ga, ua);
                            gt[rr][jj] = bf16_lo(gu);
                            up[rr][jj] = bf16_hi(gu);
                        }
                    }
                    if (decltype(fast)::value) {
                        float ex[4][4];
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                ex[rr][jj] = __builtin_amdgcn_exp2f(-gt[rr][jj] * 1.4426950408889634f);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj) ex[rr][jj] = __builtin_amdgcn_rcpf(1.0f + ex[rr][jj]);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                a[rr][jj] = ((gt[rr][jj] * ex[rr][jj]) * up[rr][jj]) * wr[rr];
                    } else {
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                            for (int jj = 0; jj < 4; ++jj)
                                a[rr][jj] = ((gt[rr][jj] / (1.0f + expf(-gt[rr][jj]))) * up[rr][jj]) * wr[rr];
                    }
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        m[rr] = __float_as_uint(fmaxf(fmaxf(fabsf(a[rr][0]), fabsf(a[rr][1])),
                                                      fmaxf(fabsf(a[rr][2]), fabsf(a[rr][3]))));
                    group8_max_u32x4(m);
                    uint32_t codes[4], b[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        b[rr] = ue8m0_e4m3_bits(m[rr]);
                        codes[rr] = pack_fp8x4_scaled(a[rr][0], a[rr][1], a[rr][2], a[rr][3], b[rr]);
                    }
                    // the byte of row rsel (lanes rsel < 4 store it): one shift of
                    // the four bytes packed in a word instead of a select chain
                    const uint32_t b4 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
                    const uint32_t bsel = b4 >> bshift;
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        __builtin_amdgcn_raw_buffer_store_b32(codes[rr], q_rs, q_lane + I * (32 * i + 8 * rq + rr),
                                                              0, kStoreNT);
                    // group G is byte (0, 2, 1, 3)[G] of the word; lanes with
                    // rsel >= 4 store nothing (an offset past the range)
                    const int s_off = rsel < 4 ? (lrow0 + rsel) * 4 + gbyte : 0x40000000;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)bsel, s_rs, s_off, 0, 0);
                }
            }
        };
        if (g.fast_math)
            rows(std::true_type{}, std::true_type{});
        else
            rows(std::false_type{}, std::true_type{});
    }
    };

    // The epilogue of a finished narrow tile (NA row tiles hold rows): every
    // wave holds rows 0-63 of its two column tiles, acc[i][0] and acc[i][1].
    auto epilogue_n = [&](const int row0, const int nrows, const int nt, const float* s_w, auto na) __attribute__((always_inline)) {
        constexpr int NA = decltype(na)::value;
        const int lane = late_copy(tid & 63);
        const int h = lane >> 5, l32 = lane & 31;
        if (MODE == kL2) {
            // output columns 64*wid + 2*l32 + {0, 1}: one bf16 pair per row
            const int N = g.N;
            uint8_t* out_base = reinterpret_cast<uint8_t*>(g.out + (int64_t)row0 * N + nt * kBN);  // wave-uniform
            const __amdgpu_buffer_rsrc_t out_rs = rows_rsrc(out_base, nrows * N * 2);
            const int col = 64 * wid + 2 * l32;
#pragma unroll
            for (int i = 0; i < NA; ++i) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float c0, c1;
                    asm("v_accvgpr_read_b32 %0, %1" : "=v"(c0) : "a"(acc[i][0][r]));
                    asm("v_accvgpr_read_b32 %0, %1" : "=v"(c1) : "a"(acc[i][1][r]));
                    const int lrow = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(c0, c1), out_rs, 2 * (lrow * N + col), 0, kStoreNT);
                }
            }
        } else {
            // activation column 32*wid + l32 of the tile's 128: quantisation
            // group wid spans the 32 lanes of a half-wave (one row each)
            const int I = g.I;
            uint8_t* q_base = g.act_q + (int64_t)row0 * I + nt * 128 + 32 * wid;      // wave-uniform
            uint8_t* s_base = g.act_s + (int64_t)nt * g.act_s_step + (int64_t)row0 * 4;  // wave-uniform
            const __amdgpu_buffer_rsrc_t q_rs = rows_rsrc(q_base, nrows * I);
            const __amdgpu_buffer_rsrc_t s_rs = rows_rsrc(s_base, nrows * 4);
            const int gbyte = ((wid & 1) << 1) | (wid >> 1);  // group wid in the word's byte order
            const uint32_t bshift = 8u * (uint32_t)(l32 & 3);
#pragma unroll
            for (int i = 0; i < NA; ++i) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int lrow0 = 32 * i + 8 * rq + 4 * h;
                    const float4 w4 = *reinterpret_cast<const float4*>(s_w + lrow0);
                    const float wr[4] = {w4.x, w4.y, w4.z, w4.w};
                    float gt[4], up[4], a[4];
                    uint32_t m[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        float ga, ua;
                        asm("v_accvgpr_read_b32 %0, %1" : "=v"(ga) : "a"(acc[i][0][4 * rq + rr]));
                        asm("v_accvgpr_read_b32 %0, %1" : "=v"(ua) : "a"(acc[i][1][4 * rq + rr]));
                        const uint32_t gu = pack_bf16x2(ga, ua);
                        gt[rr] = bf16_lo(gu);
                        up[rr] = bf16_hi(gu);
                    }
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        if (g.fast_math) {
                            const float ex = __builtin_amdgcn_exp2f(-gt[rr] * 1.4426950408889634f);
                            a[rr] = ((gt[rr] * __builtin_amdgcn_rcpf(1.0f + ex)) * up[rr]) * wr[rr];
                        } else {
                            a[rr] = ((gt[rr] / (1.0f + expf(-gt[rr]))) * up[rr]) * wr[rr];
                        }
                        m[rr] = __float_as_uint(fabsf(a[rr]));
                    }
                    group32_max_u32x4(m);
                    uint32_t b[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        b[rr] = ue8m0_e4m3_bits(m[rr]);
                        const uint32_t code = pack_fp8x2_scaled(a[rr], 0.f, b[rr]);
                        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, q_rs, (lrow0 + rr) * I + l32, 0, kStoreNT);
                    }
                    // lanes l32 = 0..3 store the scale byte of rows lrow0 + l32
                    const uint32_t b4 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
                    const int s_off = l32 < 4 ? (lrow0 + l32) * 4 + gbyte : 0x40000000;
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(b4 >> bshift), s_rs, s_off, 0, 0);
                }
            }
        }
    };

    // ---- main loop: three LDS stages, sub-step pipelined operands ---------
    // X holds sub-step 0 and Y sub-step 1 of the current step k.  While the 16
    // MFMAs of X run, Y is read from step k's stage and the second half of
    // step k+2's loads goes out.  Then each wave waits for its own loads of
    // step k+1 (the newest 14 loads may still fly) and meets the others at a
    // barrier: step k+1's stage is complete and step k's stage is free (all
    // its reads are done), so the first half of step k+3's loads goes into it
    // beside the MFMAs of Y, while X is read from step k+1's stage.  Loads go
    // out one per two MFMAs, so the load path never backs up the MFMA issue
    // and LDS writes are spread evenly over the step.  Every MFMA is fenced
    // together with the reads/loads issued beside it, so the compiler keeps
    // this order; the loop body is branch-free.  (A wave issues at most one
    // instruction per 4 cycles, so each 64-cycle MFMA leaves room for about
    // 15 others: the loop keeps every window under that.)
    // First loads of a tile: its routing weights (L1), steps 0 and 1 and the
    // first half of step 2 -- 35 loads per wave (36 with the weights).  The
    // wait leaves the newest 21 in flight: the weights and step 0 have landed
    // (loads complete in order; stores issued in between only make the wait
    // longer).
    auto issue_weights = [&](float* sw) __attribute__((always_inline)) {
        if (MODE == kL1) dma_x1(lds_addr(sw) + w_dst4, g.pool_w + row0, (uint32_t)(tid * 4));
    };
    auto prologue = [&](float* sw) __attribute__((always_inline)) {
        issue_weights(sw);
        issue_half(lds_addr(cur), 0, 0, nar_sel);
        issue_half(lds_addr(cur), 0, 1, nar_sel);
        if (nk > 1) {
            issue_half(lds_addr(next), 1, 0, nar_sel);
            issue_half(lds_addr(next), 1, 1, nar_sel);
        }
        if (nk > 2) issue_half(lds_addr(third), 2, 0, nar_sel);
    };
    auto wait_prologue = [&]() __attribute__((always_inline)) {
        if (nk > 2)
            barrier_after_vmcnt21();
        else if (nk > 1)
            barrier_after_vmcnt14();
        else
            barrier_after_vmcnt0();
    };
    float* s_w = s_wa;
    float* s_w_next = s_wb;
    lnar = nrows <= kNarrowRows ? 1 : 0;
    prologue(s_w);
    wait_prologue();
    // Two instantiations of the tile loop: SEAM (nk >= 3) runs the K-step
    // stream on across tiles; otherwise the next tile's prologue goes out
    // after the K loop.  (One loop with both tails inside makes the register
    // allocator spill the operand fragments.)
    auto tile_loop = [&](auto seam) __attribute__((always_inline)) {
    constexpr bool SEAM = decltype(seam)::value;
    for (;;) {
    const int lg_next = logical + nj;
    const bool more = lg_next < t_hi;
    auto rotate = [&]() __attribute__((always_inline)) {
        const uint8_t* t = cur;
        cur = next;
        next = third;
        third = t;
    };
    // L1: the next tile's token indices arrive in s_tok by a direct load
    // issued at this tile's start (below).  Every wave has waited for its
    // own by the barrier of step 1 (the loads of step 3 are the newest 14
    // then), so from step 2 on any wave may read them; with nk = 3 or 4 the
    // loop reaches its last three steps before that, and one extra wait
    // stands in.  Reading them gives the next tile's load offsets, which take
    // over where the scalar bases switch.
    auto prep_next_offsets = [&]() __attribute__((always_inline)) {
        if constexpr (MODE == kL1) {
            if (nk == 3)
                barrier_after_vmcnt0();
            else if (nk == 4)
                barrier_after_vmcnt14();
            gather_offsets([&](int r) { return s_tok[r]; }, nlo);
        }
    };
    auto switch_offsets = [&](bool sw) __attribute__((always_inline)) {
        if constexpr (MODE == kL1) {
            lo.a0 = sw ? nlo.a0 : lo.a0;
            lo.a1 = sw ? nlo.a1 : lo.a1;
            lo.a2 = sw ? nlo.a2 : lo.a2;
            lo.a3 = sw ? nlo.a3 : lo.a3;
            lo.a4 = sw ? nlo.a4 : lo.a4;
            lo.a5 = sw ? nlo.a5 : lo.a5;
            lo.a6 = sw ? nlo.a6 : lo.a6;
            lo.a7 = sw ? nlo.a7 : lo.a7;
        }
    };
    // The K loop, for a wave with ACT row tiles holding rows; every variant
    // issues the same loads and meets the same barriers.
    auto k_loop = [&](auto act) __attribute__((always_inline)) {
        SubFrags X, Y;
        ScaleWords Wc, Wn;  // words in use (shifted), words of the next step as read
        read_all(X, Wn, cur, 0, act);
        if constexpr (SEAM) {
            // Steps k+2 and k+3 past the end of the tile are the next tile's
            // steps 0, 1, 2.  The steady loop runs while both are this
            // tile's; the last three steps run in a second loop whose scalar
            // bases switch to the next tile (by selects: no branch in the
            // body) once step nk-3 has sent its last load of this tile, beside
            // MFMA 14 of its first half.  The last tile of a workgroup loads
            // its own first steps again instead (harmless; waited for before
            // the workgroup ends).  The barrier of step nk-1 waits for the next
            // tile's step 0, which its second half reads (unused).
            int k = 0;
            for (; k + 3 < nk; ++k) {
                const uint32_t dst2 = lds_addr(third);
    #pragma unroll
                for (int g = 0; g < 16; ++g) {
                    shift_for(Wc, Wn, g, act);
                    mfma_one(X, Wc, sub0, g, act);
                    read_piece(Y, cur, 1, g, act);
                    issue_spread(dst2, k + 2, 1, g, nar_full);
                    __builtin_amdgcn_sched_barrier(0);
                }
                barrier_after_vmcnt14();
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t dst3 = lds_addr(cur);
    #pragma unroll
                for (int g = 0; g < 16; ++g) {
                    mfma_one(Y, Wc, sub1, g, act);
                    read_piece_and_scales(X, Wn, next, g, act);
                    issue_spread(dst3, k + 3, 0, g, nar_full);
                    __builtin_amdgcn_sched_barrier(0);
                }
                rotate();
            }
            prep_next_offsets();
            const MTile nrec = s_tiles[more ? tile_i + 1 : tile_i];
            const int n_e = __builtin_amdgcn_readfirstlane(nrec.expert);
            const int n_row0 = __builtin_amdgcn_readfirstlane(nrec.row0);
            const int n_nrows = __builtin_amdgcn_readfirstlane(nrec.nrows);
            const int n_nt = __builtin_amdgcn_readfirstlane(nrec.pad);
            lnar = 0;  // this tile is full
            for (; k < nk; ++k) {
                const int s2 = k + 2 < nk ? k + 2 : k + 2 - nk;
                const uint32_t dst2 = lds_addr(third);
    #pragma unroll
                for (int g = 0; g < 16; ++g) {
                    shift_for(Wc, Wn, g, act);
                    mfma_one(X, Wc, sub0, g, act);
                    if (g == 14) {
                        __builtin_amdgcn_sched_barrier(0);
                        const bool sw = k == nk - 3;
                        e = sw ? n_e : e;
                        row0 = sw ? n_row0 : row0;
                        nrows = sw ? n_nrows : nrows;
                        nt = sw ? n_nt : nt;
                        lnar = sw ? (n_nrows <= kNarrowRows ? 1 : 0) : lnar;
                        set_bases();
                        switch_offsets(sw);
                    }
                    read_piece(Y, cur, 1, g, act);
                    issue_spread(dst2, s2, 1, g, nar_sel);
                    __builtin_amdgcn_sched_barrier(0);
                }
                barrier_after_vmcnt14();
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t dst3 = lds_addr(cur);
    #pragma unroll
                for (int g = 0; g < 16; ++g) {
                    mfma_one(Y, Wc, sub1, g, act);
                    read_piece_and_scales(X, Wn, next, g, act);
                    issue_spread(dst3, k + 3 - nk, 0, g, nar_sel);
                    __builtin_amdgcn_sched_barrier(0);
                }
                rotate();
            }
        } else {
            // nk < 3: no step issues loads; the next tile's prologue goes out
            // after the K loop.
            for (int k = 0; k < nk; ++k) {
    #pragma unroll
                for (int g = 0; g < 16; ++g) {
                    shift_for(Wc, Wn, g, act);
                    mfma_one(X, Wc, sub0, g, act);
                    read_piece(Y, cur, 1, g, act);
                    __builtin_amdgcn_sched_barrier(0);
                }
                barrier_after_vmcnt0();
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int g = 0; g < 16; ++g) {
                    mfma_one(Y, Wc, sub1, g, act);
                    read_piece_and_scales(X, Wn, next, g, act);  // on the last step: a stale stage, unused
                    __builtin_amdgcn_sched_barrier(0);
                }
                rotate();
            }
        }
    };
    // The K loop of a narrow tile with NA (1 or 2) row tiles holding rows:
    // 2*NA MFMAs per sub-step, the same 14 loads per step and the same
    // barriers as a full tile, so the two kinds of tile chain freely.  Read r
    // of a sub-step goes beside MFMA r*NM/RP, load piece p of a half beside
    // MFMA p*NM/7.
    auto k_loop_n = [&](auto na) __attribute__((always_inline)) {
        constexpr int NA = decltype(na)::value;
        constexpr int NM = 2 * NA;
        constexpr int RP = NA == 2 ? 6 : 4;
        SubFrags X, Y;
        ScaleWords Wc, Wn;
        auto reads_beside = [&](SubFrags& f, const uint8_t* base, int s, int q) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < RP; ++r)
                if (r * NM / RP == q) read_piece_n(f, base, s, r);
        };
        auto loads_beside = [&](uint32_t st, int kk, int hf, int q, auto nar) __attribute__((always_inline)) {
#pragma unroll
            for (int p = 0; p < 7; ++p)
                if (p * NM / 7 == q) issue_piece(st, kk, 7 * hf + p, nar);
        };
#pragma unroll
        for (int r = 0; r < RP; ++r) read_piece_n(X, cur, 0, r);
        read_scales_n(Wn, cur);
        if constexpr (SEAM) {
            // as in k_loop: a steady loop, then the last three steps, whose
            // loads past the tile's end are the next tile's first steps
            int k = 0;
            for (; k + 3 < nk; ++k) {
                const uint32_t dst2 = lds_addr(third);
    #pragma unroll
                for (int q = 0; q < NM; ++q) {
                    if (q == 0) shift_n(Wc, Wn);
                    mfma_n(X, Wc, sub0, q);
                    reads_beside(Y, cur, 1, q);
                    loads_beside(dst2, k + 2, 1, q, nar_narrow);
                    __builtin_amdgcn_sched_barrier(0);
                }
                barrier_after_vmcnt14();
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t dst3 = lds_addr(cur);
    #pragma unroll
                for (int q = 0; q < NM; ++q) {
                    mfma_n(Y, Wc, sub1, q);
                    reads_beside(X, next, 0, q);
                    if (q == 0) read_scales_n(Wn, next);
                    loads_beside(dst3, k + 3, 0, q, nar_narrow);
                    __builtin_amdgcn_sched_barrier(0);
                }
                rotate();
            }
            prep_next_offsets();
            const MTile nrec = s_tiles[more ? tile_i + 1 : tile_i];
            const int n_e = __builtin_amdgcn_readfirstlane(nrec.expert);
            const int n_row0 = __builtin_amdgcn_readfirstlane(nrec.row0);
            const int n_nrows = __builtin_amdgcn_readfirstlane(nrec.nrows);
            const int n_nt = __builtin_amdgcn_readfirstlane(nrec.pad);
            lnar = 1;  // this tile is narrow
            for (; k < nk; ++k) {
                const int s2 = k + 2 < nk ? k + 2 : k + 2 - nk;
                const uint32_t dst2 = lds_addr(third);
    #pragma unroll
                for (int q = 0; q < NM; ++q) {
                    if (q == 0) shift_n(Wc, Wn);
                    mfma_n(X, Wc, sub0, q);
                    reads_beside(Y, cur, 1, q);
                    loads_beside(dst2, s2, 1, q, nar_sel);
                    __builtin_amdgcn_sched_barrier(0);
                }
                {
                    // this half's loads are out: switch to the next tile
                    const bool sw = k == nk - 3;
                    e = sw ? n_e : e;
                    row0 = sw ? n_row0 : row0;
                    nrows = sw ? n_nrows : nrows;
                    nt = sw ? n_nt : nt;
                    lnar = sw ? (n_nrows <= kNarrowRows ? 1 : 0) : lnar;
                    set_bases();
                    switch_offsets(sw);
                }
                barrier_after_vmcnt14();
                __builtin_amdgcn_sched_barrier(0);
                const uint32_t dst3 = lds_addr(cur);
    #pragma unroll
                for (int q = 0; q < NM; ++q) {
                    mfma_n(Y, Wc, sub1, q);
                    reads_beside(X, next, 0, q);
                    if (q == 0) read_scales_n(Wn, next);
                    loads_beside(dst3, k + 3 - nk, 0, q, nar_sel);
                    __builtin_amdgcn_sched_barrier(0);
                }
                rotate();
            }
        } else {
            for (int k = 0; k < nk; ++k) {
    #pragma unroll
                for (int q = 0; q < NM; ++q) {
                    if (q == 0) shift_n(Wc, Wn);
                    mfma_n(X, Wc, sub0, q);
                    reads_beside(Y, cur, 1, q);
                    __builtin_amdgcn_sched_barrier(0);
                }
                barrier_after_vmcnt0();
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int q = 0; q < NM; ++q) {
                    mfma_n(Y, Wc, sub1, q);
                    reads_beside(X, next, 0, q);  // on the last step: a stale stage, unused
                    if (q == 0) read_scales_n(Wn, next);
                    __builtin_amdgcn_sched_barrier(0);
                }
                rotate();
            }
        }
    };
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int c_row0 = row0, c_nrows = nrows, c_nt = nt;
    const bool c_narrow = nrows <= kNarrowRows;
    if constexpr (MODE == kL1) {
        // the next tile's token indices (this tile's again on the last one)
        const int nrow0 = __builtin_amdgcn_readfirstlane(s_tiles[more ? tile_i + 1 : tile_i].row0);
        dma_x1(lds_addr(s_tok) + w_dst4, g.pool_tok + nrow0, (uint32_t)(tid * 4));
    }
    // (L2 only: a short L1 tile is bound by its loads, and the variants cost
    // the L1 kernel registers)
    const int nact = MODE == kL1 ? 2 : (nrows > 64 * wm + 32 ? 2 : (nrows > 64 * wm ? 1 : 0));
    if (c_narrow) {
        if (nrows > 32)
            k_loop_n(std::integral_constant<int, 2>{});
        else
            k_loop_n(std::integral_constant<int, 1>{});
    } else if (nact == 2) {
        k_loop(std::integral_constant<int, 2>{});
    } else if (nact == 1) {
        k_loop(std::integral_constant<int, 1>{});
    } else {
        k_loop(std::integral_constant<int, 0>{});
    }

    if (SEAM) {
        // the next tile's routing weights (L1); its step 0 is waited for
        // after the epilogue, leaving its step 1, the first half of step 2
        // and the weights in flight
        issue_weights(s_w_next);
    } else if (more) {
        // once every wave is done reading the stages, the next tile's first
        // loads go out, then this tile's epilogue runs while they fly
        take(s_tiles[tile_i + 1]);
        set_bases();
        lnar = nrows <= kNarrowRows ? 1 : 0;
        if constexpr (MODE == kL1) {
            // the K loop's barriers have waited for the token indices
            gather_offsets([&](int r) { return s_tok[r]; }, nlo);
            switch_offsets(true);
        }
        lds_reads_done_barrier();
        prologue(s_w_next);
    }
    if (!c_narrow)
        epilogue(c_row0, c_nrows, c_nt, s_w);
    else if (c_nrows > 32)
        epilogue_n(c_row0, c_nrows, c_nt, s_w, std::integral_constant<int, 2>{});
    else
        epilogue_n(c_row0, c_nrows, c_nt, s_w, std::integral_constant<int, 1>{});
    if (!more) break;
    if (SEAM && MODE == kL1)
        barrier_after_vmcnt22();
    else
        wait_prologue();
    float* t = s_w;
    s_w = s_w_next;
    s_w_next = t;
    logical = lg_next;
    ++tile_i;
    }
    };
    if (nk >= 3)
        tile_loop(std::true_type{});
    else
        tile_loop(std::false_type{});
    wait_all_loads();
}

// ---- decode-shaped GEMMs -------------------------------------------------
// For batches whose experts hold few rows (at most kDecRows on average, e.g.
// 128 tokens x 8 slots over 32 experts): the weights stream through once and
// the bytes each CU keeps in flight set the speed (the page "Normal vs
// Low-Latency", sections 5 and 10, names such a low-latency mode with a
// shallower pipeline).  Here: tiles of at most 64 rows x 256 columns, one
// workgroup per (tile, n-tile) -- no persistence, no cross-tile seam -- and
// three LDS stages of 26 KB, so two workgroups share a CU and each keeps two
// K steps of loads in flight while it multiplies the third.  The waves split
// the columns as the narrow tiles of the persistent kernel do (b_row_narrow:
// wave w has gate and up of quantisation group w in L1, column pairs in
// L2), each covering rows 0-63 (two 32-row MFMA tiles): the same MFMAs in
// the same K order for every output as there, hence the same results.
// Loads per wave and K step: 2 A chunks of 1 KB, 4 B chunks of 1 KB, the
// 64 rows' A-scale words (into the wave's own copy) and 64 of the 256 B-scale
// words, all direct global->LDS.  With sa_by_token, L1 takes its rows'
// A-scale words from the token-major words by token (GemmArgs SA = those
// words, sa_step = 4), so the call needs no pool copy of them; as those are
// 64 scattered words, wave 0 alone fetches them into a copy all waves read.
// B_NT: the weight codes and scale words are loaded with the non-temporal
// hint (the L1 kernel for tile-blocked weights).
template <int MODE, int RM, bool B_NT = false>
__device__ __forceinline__ void gemm_decode(const GemmArgs& g, uint8_t* lds, float* s_w) {
    constexpr int ROWS = dec_rows(RM);         // tile rows: 2 RM MFMA row tiles per wave
    constexpr int STAGES = dec_stages(RM);
    constexpr int SA_BYTES = dec_stage_a(RM);
    constexpr int SB_OFF = SA_BYTES + kDecStageB;            // A-scale copies
    constexpr int SBW_OFF = SB_OFF + dec_stage_sa(RM);       // B-scale words
    constexpr int STAGE_BYTES = dec_stage_bytes(RM);
    constexpr int LPS = 2 * RM + 4 + RM + 1;   // loads per wave and K step
    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5, l32 = lane & 31;
    const int tile = (int)blockIdx.x / g.ntiles;
    const int nt = (int)blockIdx.x - tile * g.ntiles;
    if (tile >= *g.num_mtiles) return;
    const MTile rec = g.mtiles[tile];
    const int e = __builtin_amdgcn_readfirstlane(rec.expert);
    const int row0 = __builtin_amdgcn_readfirstlane(rec.row0);
    const int nrows = __builtin_amdgcn_readfirstlane(rec.nrows);
    const int Kdim = g.Kdim, nk = Kdim / kBK, b_ld = Kdim / 2;
    // 32-row MFMA row tiles that hold rows of this tile (wave-uniform): the
    // others skip their MFMAs and epilogue.  (Their A rows are still loaded:
    // a 4-byte stand-in load instead made the T = 128 L1 3 % slower.)
    const int nrt = (nrows + 31) >> 5;

    // per-lane load offsets
    // A: chunk q = tid + 256 i (i < 2 RM) is LDS row q/8, physical chunk q%8
    // holding logical chunk (q%8) ^ ((row/2)%8); L1 rows come from the
    // token-major codes through pool_tok (indices clamped into the buffer).
    uint32_t a_off[2 * RM];
    {
        const uint32_t tmax = (uint32_t)(g.T - 1);
#pragma unroll
        for (int i = 0; i < 2 * RM; ++i) {
            const int row = (tid >> 3) + 32 * i;
            const int lch = (tid & 7) ^ ((row >> 1) & 7);
            const uint32_t arow = MODE == kL1 ? min((uint32_t)g.pool_tok[row0 + row], tmax) : (uint32_t)row;
            a_off[i] = arow * (uint32_t)Kdim + 16u * (uint32_t)lch;
        }
    }
    // B: chunk q = tid + 256 i (i = 0..3) is LDS row q/4 (weight row
    // b_row_narrow of it), physical chunk q%4 holding logical (q%4) ^ ((row/4)%4)
    const int brow0 = b_row_narrow<MODE>(nt, 0, g.I);
    // tile-blocked codes: rows 64 bytes apart, L1's up rows right after its
    // 128 gate rows, 16 KiB per K step
    const int b_rs = g.b_tiled ? kBK / 2 : b_ld, bI = g.b_tiled ? 128 : g.I;
    const int64_t b_ks = g.b_tiled ? (int64_t)kBTileBytes : kBK / 2;
    auto boff = [&](int i) {
        const int row = (tid >> 2) + 64 * i;
        const int lch = (tid & 3) ^ ((row >> 2) & 3);
        return (uint32_t)((b_row_narrow<MODE>(0, row, bI) - b_row_narrow<MODE>(0, 0, bI)) * b_rs + 16 * lch);
    };
    const uint32_t b_off0 = boff(0), b_off1 = boff(1), b_off2 = boff(2), b_off3 = boff(3);
    // scale words: A rows row0 + lane (+ 64) into the wave's copy -- L1 with
    // sa_by_token straight from the token-major words of its token (no pool
    // copy of them), else from the packed k-major words of the pool rows;
    // B: LDS word tid is the word of LDS B row tid
    const bool sa_tok = RM == 1 && MODE == kL1 && g.sa_by_token;
    uint32_t sa_off;
    if (sa_tok)
        sa_off = 4u * min((uint32_t)g.pool_tok[row0 + lane], (uint32_t)(g.T - 1)) * (uint32_t)nk;
    else
        sa_off = 4u * (uint32_t)lane;
    const uint32_t sb_off = (uint32_t)(4 * (b_row_narrow<MODE>(nt, tid, g.I) - brow0));
    const uint8_t* a_base = MODE == kL1 ? g.A : g.A + (int64_t)row0 * Kdim;
    const uint8_t* b_base = g.b_tiled ? g.B + ((int64_t)e * g.ntiles + nt) * (int64_t)nk * kBTileBytes
                                      : g.B + ((int64_t)e * g.N + brow0) * b_ld;
    const uint8_t* sa_base = sa_tok ? g.SA : g.SA + (int64_t)row0 * 4;  // by token: token-major words
    const int64_t sb_step = (int64_t)g.N * 4;
    const uint8_t* sb_base = g.SB + (int64_t)e * nk * sb_step + (int64_t)brow0 * 4;

    if (MODE == kL1 && tid < ROWS) s_w[tid] = g.pool_w[row0 + tid];  // rows past the tile: unused

    auto stage = [&](int k) { return lds + (k % STAGES) * STAGE_BYTES; };
    auto issue = [&](int k) __attribute__((always_inline)) {
        const uint32_t st = lds_addr(stage(k));
        const uint32_t wa = st + 1024u * wid;
#pragma unroll
        for (int i = 0; i < 2 * RM; ++i) {
            dma_x4(wa + 4096u * i, a_base + k * kBK, a_off[i]);
        }
        // L1's tile-blocked weights with the non-temporal hint: each K step
        // reads whole lines of a contiguous block once (measured at T = 128:
        // L1 92.7 -> 87 us, and L2 51.8 -> 45.4 us, whose weights then stay
        // in the Infinity Cache from one call to the next; the hint on L2's
        // weights: L2 51.4 -> 60 us; on the as-given layout, where a K step
        // reads half of each line and the next step the other half, the step
        // 0.213 -> 0.257 ms)
        const uint32_t wb = st + SA_BYTES + 1024u * wid;
        auto bload = [&](uint32_t dst, uint32_t off) __attribute__((always_inline)) {
            if (B_NT)
                dma_x4_nt(dst, b_base + k * b_ks, off);
            else
                dma_x4(dst, b_base + k * b_ks, off);
        };
        bload(wb, b_off0);
        bload(wb + 4096, b_off1);
        bload(wb + 8192, b_off2);
        bload(wb + 12288, b_off3);
        const uint32_t wsa = st + SB_OFF + 4u * ROWS * wid;
        if (sa_tok) {
            // the rows' words scattered by token: wave 0 fetches them into
            // the shared copy; the other waves keep the per-wave count of
            // loads with a contiguous stand-in (the B words again) into
            // their own unused slot
            if (wid == 0)
                dma_x1(st + SB_OFF, sa_base + k * g.sa_step, sa_off);
            else
                dma_x1(wsa, sb_base + k * sb_step, sb_off);
        } else {
#pragma unroll
            for (int i = 0; i < RM; ++i) dma_x1(wsa + 256u * i, sa_base + k * g.sa_step, sa_off + 256u * i);
        }
        if (B_NT)
            dma_x1_nt(st + SBW_OFF + 256u * wid, sb_base + k * sb_step, sb_off);
        else
            dma_x1(st + SBW_OFF + 256u * wid, sb_base + k * sb_step, sb_off);
    };

    // this wave's column tiles (b_row_narrow): L1 gate and up of group wid,
    // L2 the column pair 2 wid, 2 wid + 1
    const int jn0 = MODE == kL1 ? wid : 2 * wid;
    const int jn1 = MODE == kL1 ? wid + 4 : 2 * wid + 1;
    const int a_sw = (l32 >> 1) & 7, b_sw = (l32 >> 2) & 3;
    const int hs = 16 * h;
    v16f acc[2 * RM][2];
#pragma unroll
    for (int i = 0; i < 2 * RM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    constexpr int kAhead = STAGES - 1;  // K steps whose loads are in flight
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
        if (k < nk) issue(k);
    for (int k = 0; k < nk; ++k) {
        // step k's loads have landed (the later steps' may still fly: LPS
        // loads per step and wave), and every wave is done reading step
        // k-1's stage, which step k + kAhead then refills
        const int later = min(kAhead - 1, nk - 1 - k);
        if (later >= 2)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LPS) : "memory");
        else if (later == 1)
            asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LPS) : "memory");
        else
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (k + kAhead < nk) issue(k + kAhead);
        const uint8_t* sA = stage(k);
        const uint8_t* sB = sA + SA_BYTES;
        const uint8_t* sSA = sA + SB_OFF + (sa_tok ? 0 : 4 * ROWS * wid);  // by token: wave 0's copy
        const uint8_t* sSB = sA + SBW_OFF;
        int wa[2 * RM];
#pragma unroll
        for (int i = 0; i < 2 * RM; ++i)
            wa[i] = (int)(*reinterpret_cast<const uint32_t*>(sSA + 4 * (32 * i + l32)) >> hs);
        int wb0 = *reinterpret_cast<const int*>(sSB + 4 * (32 * jn0 + l32));
        int wb1 = *reinterpret_cast<const int*>(sSB + 4 * (32 * jn1 + l32));
        wb0 = (int)((uint32_t)wb0 >> hs);
        wb1 = (int)((uint32_t)wb1 >> hs);
        auto sub = [&](auto sconst) __attribute__((always_inline)) {
            constexpr int S = decltype(sconst)::value;
            v8i b[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const uint8_t* rowp = sB + (32 * (jj ? jn1 : jn0) + l32) * (kBK / 2);
                const uint4 v = *reinterpret_cast<const uint4*>(rowp + 16 * ((2 * S + h) ^ b_sw));
                b[jj] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < 2 * RM; ++i) {
                if (i >= nrt) continue;  // no rows
                const uint8_t* rowp = sA + (32 * i + l32) * kBK;
                const uint4 v0 = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * S + h) ^ a_sw));
                const uint4 v1 = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * S + 2 + h) ^ a_sw));
                const v8i a = v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        a, b[jj], acc[i][jj], 0, 4, S, wa[i], S, jj ? wb1 : wb0);
            }
        };
        sub(std::integral_constant<int, 0>{});
        sub(std::integral_constant<int, 1>{});
    }
    wait_all_loads();

    // epilogue (as for the narrow tiles of the persistent kernel): rows past
    // the tile's end are dropped by the buffer range
    if (MODE == kL2) {
        const int N = g.N;
        uint8_t* out_base = reinterpret_cast<uint8_t*>(g.out + (int64_t)row0 * N + nt * kBN);
        const __amdgpu_buffer_rsrc_t out_rs = rows_rsrc(out_base, nrows * N * 2);
        const int col = 64 * wid + 2 * l32;
#pragma unroll
        for (int i = 0; i < 2 * RM; ++i) {
            if (i >= nrt) continue;  // no rows
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int lrow = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                __builtin_amdgcn_raw_buffer_store_b32(pack_bf16x2(acc[i][0][r], acc[i][1][r]), out_rs,
                                                      2 * (lrow * N + col), 0, kStoreDecode);
            }
        }
    } else {
        const int I = g.I;
        uint8_t* q_base = g.act_q + (int64_t)row0 * I + nt * 128 + 32 * wid;
        uint8_t* s_base = g.act_s + (int64_t)nt * g.act_s_step + (int64_t)row0 * 4;
        const __amdgpu_buffer_rsrc_t q_rs = rows_rsrc(q_base, nrows * I);
        const __amdgpu_buffer_rsrc_t s_rs = rows_rsrc(s_base, nrows * 4);
        const int gbyte = ((wid & 1) << 1) | (wid >> 1);  // group wid in the word's byte order
        const uint32_t bshift = 8u * (uint32_t)(l32 & 3);
        __syncthreads();  // s_w visible
#pragma unroll
        for (int i = 0; i < 2 * RM; ++i) {
            if (i >= nrt) continue;  // no rows
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int lrow0 = 32 * i + 8 * rq + 4 * h;
                float gt[4], up[4], a[4];
                uint32_t m[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint32_t gu = pack_bf16x2(acc[i][0][4 * rq + rr], acc[i][1][4 * rq + rr]);
                    gt[rr] = bf16_lo(gu);
                    up[rr] = bf16_hi(gu);
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float wr = s_w[lrow0 + rr];
                    if (g.fast_math) {
                        const float ex = __builtin_amdgcn_exp2f(-gt[rr] * 1.4426950408889634f);
                        a[rr] = ((gt[rr] * __builtin_amdgcn_rcpf(1.0f + ex)) * up[rr]) * wr;
                    } else {
                        a[rr] = ((gt[rr] / (1.0f + expf(-gt[rr]))) * up[rr]) * wr;
                    }
                    m[rr] = __float_as_uint(fabsf(a[rr]));
                }
                group32_max_u32x4(m);
                uint32_t b[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    b[rr] = ue8m0_e4m3_bits(m[rr]);
                    const uint32_t code = pack_fp8x2_scaled(a[rr], 0.f, b[rr]);
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, q_rs, (lrow0 + rr) * I + l32, 0, kStoreDecode);
                }
                // lanes l32 = 0..3 store the scale byte of rows lrow0 + l32
                const uint32_t b4 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
                const int s_off = l32 < 4 ? (lrow0 + l32) * 4 + gbyte : 0x40000000;
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(b4 >> bshift), s_rs, s_off, 0, 0);
            }
        }
    }
}


// ---- L1 and L2 in one launch, the activations kept in LDS -----------------
// One workgroup per m-tile of at most kFusedRows rows of one expert (the
// second tile table).  First L1 over all 2I gate/up columns in I/128 chunks of
// 256 LDS B rows (gate and up of four quantisation groups, the narrow column
// order: wave w takes gate and up of group w), each chunk's SwiGLU / requant
// epilogue writing its 128 e4m3 activation columns -- exactly one 128-wide K
// block of L2 -- and their scale bytes into LDS; then L2 over all H output
// columns in H/256 chunks, its A operand read from that LDS tile, each
// chunk's bf16 rows stored to the pool-order output.  Every wave covers all
// rows (four 32-row MFMA tiles; those without rows skip their MFMAs) and two
// 32-column tiles, so every output gets the same MFMAs in the same K order as
// in the other GEMM kernels, hence the same bits.
//
// K steps of 64 (one MFMA sub-step): three LDS stages of 16 KiB (A 128 rows x
// 64 B, B 256 rows x 32 B) filled by direct loads two steps ahead, the stream
// running on across chunk and phase boundaries; the scale words of each
// 128-wide K block (each wave's copy of the A rows' words, and the B words)
// go to a ring of two slots with the block's first step.  Per wave and step:
// L1 7 loads on a block's first step and 4 on its second, L2 3 and 2; an L2
// chunk's epilogue issues kFusedStores stores.  The waits count them, taking
// vector memory operations to complete in issue order.
//
// Measured on one MI355X with T = 16384, H = 2048, I = 768, E = 128, K = 8:
// 1.12 ms for this launch against 0.58 ms for the two separate GEMMs.  The
// 99 KB activation tile leaves room in the 160 KiB LDS for 16 KiB stages
// only, so a barrier covers 8 MFMAs per wave (32 in the persistent GEMMs),
// and with one wave per SIMD the LDS reads, scalar work and barriers of each
// step are not hidden (1.5 k cycles per step of 512 MFMA cycles even with the
// loads taken out).  The layer offers it as a choice (gemm_tiles), not by
// default.
constexpr int kFStageA = kFusedRows * 64;
constexpr int kFStageB = kBN * 32;
constexpr int kFStage = kFStageA + kFStageB;
constexpr int kFScaleSA = 4 * kFusedRows * 4;
constexpr int kFScale = kFScaleSA + kBN * 4;
constexpr int kFusedStores = 32;
constexpr int kFusedLds = 3 * kFStage + 2 * kFScale + kFusedRows * kFusedMaxI + (kFusedMaxI / 128) * kFusedRows * 4 +
                          kFusedRows * 4;
static_assert(kFusedLds <= 160 * 1024, "LDS");

// s_waitcnt vmcnt(N) lgkmcnt(0) and a workgroup barrier.
template <int N>
__device__ __forceinline__ void waitcnt_barrier() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void gemm_fused(const GemmArgs& g1, const GemmArgs& g2, uint8_t* lds) {
    // the arguments in scalars: the loop must not read them through a
    // pointer (a generic load there waits for every direct load in flight)
    const uint8_t* const A1 = g1.A;
    const uint8_t* const SA1 = g1.SA;
    const uint8_t* const B1 = g1.B;
    const uint8_t* const SB1 = g1.SB;
    const uint8_t* const B2 = g2.B;
    const uint8_t* const SB2 = g2.SB;
    uint16_t* const OUT = g2.out;
    const int64_t sa_step1 = g1.sa_step;
    const int32_t* const pool_tok = g1.pool_tok;
    const float* const pool_w = g1.pool_w;
    const MTile* const mtiles = g1.mtiles;
    const int32_t* const num_mtiles = g1.num_mtiles;
    const int T1 = g1.T, N1 = g1.N, N2 = g2.N, ntl1 = g1.ntiles, ntl2 = g2.ntiles;
    const bool tiled1 = g1.b_tiled != 0, tiled2 = g2.b_tiled != 0, fast_math = g1.fast_math != 0;
    uint8_t* stg = lds;                                  // 3 stages
    uint8_t* scl = stg + 3 * kFStage;                    // 2 scale slots
    uint8_t* act = scl + 2 * kFScale;                    // [rows][I] e4m3, swizzled
    uint8_t* sact = act + kFusedRows * kFusedMaxI;       // words [I/128][rows]
    float* s_w = reinterpret_cast<float*>(sact + (kFusedMaxI / 128) * kFusedRows * 4);

    const int tid = threadIdx.x;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int h = lane >> 5, l32 = lane & 31;
    const int hs = 16 * h;

    // XCD-contiguous tiles: the hardware places workgroup b on XCD b % 8 and
    // XCD x takes the tiles [total*x/8, total*(x+1)/8), so the tiles of an
    // expert mostly run together on one XCD and share its weights through
    // that XCD's L2.  (The grid is a multiple of 8, at least 8 times the
    // largest share; the extra workgroups return.)
    const int total = *num_mtiles;
    const int xcd = (int)blockIdx.x & 7;
    const int tile = (int)((int64_t)total * xcd / 8) + ((int)blockIdx.x >> 3);
    if (tile >= (int)((int64_t)total * (xcd + 1) / 8)) return;
    const MTile rec = mtiles[tile];
    const int e = __builtin_amdgcn_readfirstlane(rec.expert);
    const int row0 = __builtin_amdgcn_readfirstlane(rec.row0);
    const int nrows = __builtin_amdgcn_readfirstlane(rec.nrows);
    const int nrt = (nrows + 31) >> 5;  // 32-row MFMA tiles holding rows

    const int H = g1.Kdim, I = g1.I;
    const int nkb1 = H / 128, nkb2 = I / 128;  // 128-wide K blocks per chunk
    const int nch1 = I / 128, nch2 = H / kBN;  // chunks
    const int S1 = 2 * nkb1 * nch1;            // K steps of the L1 phase
    const int ST = S1 + 2 * nkb2 * nch2;

    // ---- per-lane load offsets ---------------------------------------------
    // A (L1): chunk q = tid + 256 p (p = 0, 1) is LDS row q/4, physical chunk
    // q%4 holding logical chunk (q%4) ^ ((row/4)%4), from the token row
    // pool_tok[row0 + row] (clamped into the buffer).
    uint32_t a_off0, a_off1;
    {
        const uint32_t tmax = (uint32_t)(T1 - 1);
        const int lch = (tid & 3) ^ ((tid >> 4) & 3);
        const uint32_t t0 = min((uint32_t)pool_tok[row0 + (tid >> 2)], tmax);
        const uint32_t t1 = min((uint32_t)pool_tok[row0 + (tid >> 2) + 64], tmax);
        a_off0 = t0 * (uint32_t)H + 16u * (uint32_t)lch;
        a_off1 = t1 * (uint32_t)H + 16u * (uint32_t)lch;
    }
    // B: chunk q = tid + 256 p is LDS row q/2 (weight row b_row_narrow of it),
    // physical chunk q%2 holding logical (q%2) ^ ((row/8)%2), 32 bytes a row
    // per step.
    auto boffs = [&](auto mode, bool tiled, int kdim, int Iv, uint32_t& o0, uint32_t& o1) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode)::value;
        const int rs = tiled ? kBK / 2 : kdim / 2, bI = tiled ? 128 : Iv;
        const int lch = (tid & 1) ^ ((tid >> 4) & 1);
        const int r0 = tid >> 1, r1 = r0 + 128;
        o0 = (uint32_t)((b_row_narrow<MODE>(0, r0, bI) - b_row_narrow<MODE>(0, 0, bI)) * rs + 16 * lch);
        o1 = (uint32_t)((b_row_narrow<MODE>(0, r1, bI) - b_row_narrow<MODE>(0, 0, bI)) * rs + 16 * lch);
    };
    uint32_t b1_o0, b1_o1, b2_o0, b2_o1;
    boffs(std::integral_constant<int, kL1>{}, tiled1, H, I, b1_o0, b1_o1);
    boffs(std::integral_constant<int, kL2>{}, tiled2, I, I, b2_o0, b2_o1);
    // B scale words: LDS word tid holds the word of LDS B row tid
    const uint32_t sb1_off = (uint32_t)(4 * (b_row_narrow<kL1>(0, tid, I) - b_row_narrow<kL1>(0, 0, I)));
    const uint32_t sb2_off = (uint32_t)(4 * (b_row_narrow<kL2>(0, tid, H) - b_row_narrow<kL2>(0, 0, H)));
    const int64_t b1_ks = tiled1 ? (int64_t)kBTileBytes : kBK / 2;
    const int64_t b2_ks = tiled2 ? (int64_t)kBTileBytes : kBK / 2;
    // scalar bases of chunk c
    auto b1_base = [&](int c) __attribute__((always_inline)) {
        return tiled1 ? B1 + ((int64_t)e * ntl1 + c) * (int64_t)nkb1 * kBTileBytes
                          : B1 + ((int64_t)e * N1 + b_row_narrow<kL1>(c, 0, I)) * (H / 2);
    };
    auto b2_base = [&](int c) __attribute__((always_inline)) {
        return tiled2 ? B2 + ((int64_t)e * ntl2 + c) * (int64_t)nkb2 * kBTileBytes
                          : B2 + ((int64_t)e * N2 + b_row_narrow<kL2>(c, 0, H)) * (I / 2);
    };
    auto sb1_base = [&](int c) __attribute__((always_inline)) {
        return SB1 + (int64_t)e * nkb1 * ((int64_t)N1 * 4) + (int64_t)b_row_narrow<kL1>(c, 0, I) * 4;
    };
    auto sb2_base = [&](int c) __attribute__((always_inline)) {
        return SB2 + (int64_t)e * nkb2 * ((int64_t)N2 * 4) + (int64_t)b_row_narrow<kL2>(c, 0, H) * 4;
    };
    const uint8_t* sa_base = SA1 + (int64_t)row0 * 4;

    if (tid < kFusedRows) s_w[tid] = pool_w[row0 + tid];  // rows past the tile: unused

    // ---- loads, in a cursor advanced per step ----------------------------
    // Running scalar pointers of the next step to load (A rows, B rows, A
    // and B scale words of its K block), moved by constant strides and set
    // afresh only at a chunk's end.
    int lu = 0, lc = 0, lissued = 0;  // step inside the chunk, chunk, steps loaded
    bool lp2 = false;                  // the next step to load is in the L2 phase
    const uint8_t *la = A1, *lb = nullptr, *lsa = sa_base, *lsb = nullptr;
    const int64_t sb1_step = (int64_t)N1 * 4, sb2_step = (int64_t)N2 * 4;
    auto set_chunk = [&]() __attribute__((always_inline)) {
        if (!lp2) {
            la = A1;
            lsa = sa_base;
            lb = b1_base(lc);
            lsb = sb1_base(lc);
        } else {
            lb = b2_base(lc);
            lsb = sb2_base(lc);
        }
    };
    set_chunk();
    const uint32_t stg0 = lds_addr(stg), scl0 = lds_addr(scl);
    uint32_t lst = stg0;   // stage of the next load
    uint32_t lsc = scl0;   // scale slot of its K block
    auto issue_next = [&]() __attribute__((always_inline)) {
        const uint32_t wa = lst + 1024u * wid, wb = lst + kFStageA + 1024u * wid;
        const bool first = (lu & 1) == 0;  // the K block's first step: its scale words
        if (!lp2) {
            dma_x4(wa, la, a_off0);
            dma_x4(wa + 4096, la, a_off1);
            dma_x4(wb, lb, b1_o0);
            dma_x4(wb + 4096, lb, b1_o1);
            if (first) {
                dma_x1(lsc + 512u * wid, lsa, 4u * lane);
                dma_x1(lsc + 512u * wid + 256u, lsa, 4u * lane + 256u);
                dma_x1(lsc + kFScaleSA + 256u * wid, lsb, sb1_off);
            }
        } else {
            dma_x4(wb, lb, b2_o0);
            dma_x4(wb + 4096, lb, b2_o1);
            if (first) dma_x1(lsc + kFScaleSA + 256u * wid, lsb, sb2_off);
        }
        ++lissued;
        lst = lst == stg0 + 2 * kFStage ? stg0 : lst + kFStage;
        if (!first) lsc = lsc == scl0 ? scl0 + kFScale : scl0;  // the block's last step
        if (++lu == 2 * (lp2 ? nkb2 : nkb1)) {
            lu = 0;
            if (!lp2) {
                if (++lc == nch1) lc = 0, lp2 = true;
            } else {
                ++lc;
            }
            if (lissued < ST) set_chunk();
        } else if (first) {
            la += 64;
            lb += 32;
        } else {
            la += 64;
            lb += (lp2 ? b2_ks : b1_ks) - 32;
            lsa += sa_step1;
            lsb += lp2 ? sb2_step : sb1_step;
        }
    };

    v16f acc[4][2];
    auto clear = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    };
    clear();

    // MFMA operands of one K step for one wave: its four row tiles' A
    // fragments and scale words, its two column tiles' B fragments and words.
    struct Frags {
        v8i a[4];
        v4i b[2];
        int wa[4], wb[2];
    };
    Frags fa, fb;  // even and odd steps
    const int b_sw = (l32 >> 3) & 1;  // B rows: (row/8)%2 of rows 32 j + l32
    const int a_sw = (l32 >> 2) & 3;  // A stage rows: (row/4)%4
    // activation tile: element (row, column) at row * I + 128 * kb' +
    // 16 * (q ^ (row/2)%8) + column % 16, with K block kb = column / 128 (kb' =
    // kb ^ (row%2) when I/128 is even, else kb, so that rows of either parity
    // start in different halves of the banks) and chunk q = (column % 128) / 16
    const bool kb_swap = (nkb2 & 1) == 0;
    const int act_sw = (l32 >> 1) & 7;

    // Reads of step t's operands, in pieces: piece 0 the B fragments and
    // words, piece 1 + i row tile i (skipped without rows unless FULL).  L1
    // takes A from the stage (columns wid, wid + 4: gate and up of group
    // wid); L2 takes A from the activation tile at K block m, sub-step S
    // (columns 2 wid, 2 wid + 1).
    auto read_piece = [&](Frags& f, int p, bool l2, const uint8_t* sA, const uint8_t* sc, int m, int S, auto full)
        __attribute__((always_inline)) {
        const int jn0 = l2 ? 2 * wid : wid, jn1 = l2 ? 2 * wid + 1 : wid + 4;
        if (p == 0) {
            const uint8_t* sB = sA + kFStageA;
            const uint4 v0 = *reinterpret_cast<const uint4*>(sB + (32 * jn0 + l32) * 32 + 16 * (h ^ b_sw));
            const uint4 v1 = *reinterpret_cast<const uint4*>(sB + (32 * jn1 + l32) * 32 + 16 * (h ^ b_sw));
            f.b[0] = v4i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w};
            f.b[1] = v4i{(int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
            f.wb[0] = (int)(*reinterpret_cast<const uint32_t*>(sc + kFScaleSA + 4 * (32 * jn0 + l32)) >> hs);
            f.wb[1] = (int)(*reinterpret_cast<const uint32_t*>(sc + kFScaleSA + 4 * (32 * jn1 + l32)) >> hs);
            return;
        }
        const int i = p - 1;
        if (!decltype(full)::value && i >= nrt) return;
        uint4 v0, v1;
        if (!l2) {
            const uint8_t* rowp = sA + (32 * i + l32) * 64;
            v0 = *reinterpret_cast<const uint4*>(rowp + 16 * (h ^ a_sw));
            v1 = *reinterpret_cast<const uint4*>(rowp + 16 * ((2 + h) ^ a_sw));
            f.wa[i] = (int)(*reinterpret_cast<const uint32_t*>(sc + 512 * wid + 4 * (32 * i + l32)) >> hs);
        } else {
            const int kb = kb_swap ? (m ^ (l32 & 1)) : m;
            const uint8_t* rowp = act + (32 * i + l32) * I + 128 * kb;
            v0 = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * S + h) ^ act_sw));
            v1 = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * S + 2 + h) ^ act_sw));
            f.wa[i] = (int)(reinterpret_cast<const uint32_t*>(sact)[m * kFusedRows + 32 * i + l32] >> hs);
        }
        f.a[i] = v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
    };
    // the MFMAs of row tile i of a step whose operands f holds (sub-step S)
    auto mfma_tile = [&](const Frags& f, int i, auto sconst, auto full) __attribute__((always_inline)) {
        constexpr int S = decltype(sconst)::value;
        if (!decltype(full)::value && i >= nrt) return;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const v8i b = v8i{f.b[j][0], f.b[j][1], f.b[j][2], f.b[j][3], 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], b, acc[i][j], 0, 4, S, f.wa[i], S,
                                                                        f.wb[j]);
        }
    };

    // L1 chunk c's epilogue: gate/up to bf16, silu(gate) * up * w, per-32
    // amax, UE8M0, e4m3 codes and scale bytes into the activation tile (the
    // same arithmetic as the other L1 epilogues).
    const int gbyte = ((wid & 1) << 1) | (wid >> 1);  // group wid in the word's byte order
    const uint32_t bshift = 8u * (uint32_t)(l32 & 3);
    auto epilogue_l1 = [&](int c, auto full) __attribute__((always_inline)) {
        const int q = 2 * wid + (l32 >> 4), byte = l32 & 15;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (!decltype(full)::value && i >= nrt) continue;
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int lrow0 = 32 * i + 8 * rq + 4 * h;
                float gt[4], up[4], a[4];
                uint32_t mx[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint32_t gu = pack_bf16x2(acc[i][0][4 * rq + rr], acc[i][1][4 * rq + rr]);
                    gt[rr] = bf16_lo(gu);
                    up[rr] = bf16_hi(gu);
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float wr = s_w[lrow0 + rr];
                    if (fast_math) {
                        const float ex = __builtin_amdgcn_exp2f(-gt[rr] * 1.4426950408889634f);
                        a[rr] = ((gt[rr] * __builtin_amdgcn_rcpf(1.0f + ex)) * up[rr]) * wr;
                    } else {
                        a[rr] = ((gt[rr] / (1.0f + expf(-gt[rr]))) * up[rr]) * wr;
                    }
                    mx[rr] = __float_as_uint(fabsf(a[rr]));
                }
                group32_max_u32x4(mx);
                uint32_t b[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int row = lrow0 + rr;
                    b[rr] = ue8m0_e4m3_bits(mx[rr]);
                    const uint32_t code = pack_fp8x2_scaled(a[rr], 0.f, b[rr]);
                    const int kb = kb_swap ? (c ^ (row & 1)) : c;
                    act[row * I + 128 * kb + 16 * (q ^ ((row >> 1) & 7)) + byte] = (uint8_t)code;
                }
                // lanes l32 = 0..3 write the scale byte of rows lrow0 + l32
                const uint32_t b4 = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
                if (l32 < 4) sact[4 * (c * kFusedRows + lrow0 + l32) + gbyte] = (uint8_t)(b4 >> bshift);
            }
        }
    };
    // L2 chunk c's epilogue: bf16 rows.  A lane holds two adjacent columns of
    // 16 rows per row tile; neighbouring lanes trade one of each pair of rows
    // (DPP lane ^ 1) so that each stores four adjacent columns (8 bytes) of
    // one row: kFusedStores stores per lane, rows past the tile's end dropped
    // by the buffer range.
    auto epilogue_l2 = [&](int c) __attribute__((always_inline)) {
        const int N = H;
        uint8_t* out_base = reinterpret_cast<uint8_t*>(OUT + (int64_t)row0 * N + c * kBN);
        const __amdgpu_buffer_rsrc_t out_rs = rows_rsrc(out_base, nrows * N * 2);
        const bool odd = (l32 & 1) != 0;
        const int col = 64 * wid + 2 * (l32 & ~1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int lrow = 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                const uint32_t v0 = pack_bf16x2(acc[i][0][r], acc[i][1][r]);          // row lrow
                const uint32_t v1 = pack_bf16x2(acc[i][0][r + 1], acc[i][1][r + 1]);  // row lrow + 1
                const uint32_t got = dpp_u32<kDppQuadSwap1>(odd ? v0 : v1);
                const v2i w = odd ? v2i{(int)got, (int)v1} : v2i{(int)v0, (int)got};
                const int row = lrow + (odd ? 1 : 0);
                __builtin_amdgcn_raw_buffer_store_b64(w, out_rs, 2 * (row * N + col), 0, kStoreDecode);
            }
        }
    };

    // ---- the step stream ---------------------------------------------------
    // Iteration t: wait for step t's loads (and every wave's reads of step
    // t-1's stage), load step t+2 into that stage, then step t-1's MFMAs with
    // step t's operand reads between them; a chunk's epilogue follows its last
    // MFMAs (in the iteration of the next chunk's first step, always even).
    // The newer vector memory operations at the wait: step t+1's loads (L1:
    // 7 on a K block's first step, 4 on its second; L2: 3 and 2) and the
    // stores of an L2 epilogue in either of the two previous iterations.
    issue_next();
    issue_next();
    auto stream = [&](auto full) __attribute__((always_inline)) {
        int t = 0;
        const uint8_t* sst = stg;  // stage of step t
        const uint8_t* rsc = scl;  // scale slot of its K block
        bool e1 = false, e2 = false;  // stores issued in iteration t-1, t-2
        const std::integral_constant<int, 0> s0;
        const std::integral_constant<int, 1> s1;
        auto begin = [&](auto ncst) __attribute__((always_inline)) {
            constexpr int N = decltype(ncst)::value;
            waitcnt_barrier<N>();
            if (lissued < ST) issue_next();
        };
        auto begin_l2 = [&](auto ncst) __attribute__((always_inline)) {
            constexpr int N = decltype(ncst)::value;
            if (e1 || e2)
                waitcnt_barrier<N + kFusedStores>();
            else
                waitcnt_barrier<N>();
            e2 = e1;
            e1 = false;
            if (lissued < ST) issue_next();
        };
        auto adv = [&](bool block_end) __attribute__((always_inline)) {
            ++t;
            sst = sst == stg + 2 * kFStage ? stg : sst + kFStage;
            if (block_end) rsc = rsc == scl ? scl + kFScale : scl;
        };
        // step t-1's MFMAs (operands in fm, sub-step SM) with step t's reads
        // into fr (phase l2, K block m of the chunk, sub-step SR)
        auto overlap = [&](Frags& fr, Frags& fm, bool l2, int m, auto sr, auto sm) __attribute__((always_inline)) {
            constexpr int SR = decltype(sr)::value;
            read_piece(fr, 0, l2, sst, rsc, m, SR, full);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mfma_tile(fm, i, sm, full);
                read_piece(fr, 1 + i, l2, sst, rsc, m, SR, full);
            }
        };
        const std::integral_constant<int, 7> n7;
        const std::integral_constant<int, 4> n4;
        const std::integral_constant<int, 3> n3;
        const std::integral_constant<int, 2> n2;
        const std::integral_constant<int, 0> n0;
        // the second step of an L1 K block (waits as its successor: the next
        // block's first step, or L2's at the phase end)
        auto l1_odd = [&](int m) __attribute__((always_inline)) {
            if (t + 1 == S1) begin(n3); else begin(n7);
            overlap(fb, fa, false, m, s1, s0);
            adv(true);
        };
        auto l2_odd = [&](int m) __attribute__((always_inline)) {
            if (t + 1 == ST) begin_l2(n0); else begin_l2(n3);
            overlap(fb, fa, true, m, s1, s0);
            adv(true);
        };
        auto l1_rest = [&]() __attribute__((always_inline)) {
            for (int m = 1; m < nkb1; ++m) {
                begin(n4);
                overlap(fa, fb, false, m, s0, s1);
                adv(false);
                l1_odd(m);
            }
        };
        auto l2_rest = [&]() __attribute__((always_inline)) {
            for (int m = 1; m < nkb2; ++m) {
                begin_l2(n2);
                overlap(fa, fb, true, m, s0, s1);
                adv(false);
                l2_odd(m);
            }
        };
        // L1 phase: chunk 0 starts the stream
        begin(n4);
#pragma unroll
        for (int p = 0; p < 5; ++p) read_piece(fa, p, false, sst, rsc, 0, 0, full);
        adv(false);
        l1_odd(0);
        l1_rest();
        for (int c = 1; c < nch1; ++c) {
            begin(n4);
            overlap(fa, fb, false, 0, s0, s1);
            epilogue_l1(c - 1, full);
            clear();
            adv(false);
            l1_odd(0);
            l1_rest();
        }
        // L2 phase; its first step closes L1: the last L1 MFMAs and epilogue,
        // every wave's activations in LDS, then the first L2 reads
        begin_l2(n2);
#pragma unroll
        for (int i = 0; i < 4; ++i) mfma_tile(fb, i, s1, full);
        epilogue_l1(nch1 - 1, full);
        clear();
        lds_reads_done_barrier();
#pragma unroll
        for (int p = 0; p < 5; ++p) read_piece(fa, p, true, sst, rsc, 0, 0, full);
        adv(false);
        l2_odd(0);
        l2_rest();
        for (int c = 1; c < nch2; ++c) {
            begin_l2(n2);
            overlap(fa, fb, true, 0, s0, s1);
            epilogue_l2(c - 1);
            e1 = true;
            clear();
            adv(false);
            l2_odd(0);
            l2_rest();
        }
        // the last step's MFMAs and the last L2 chunk's epilogue
#pragma unroll
        for (int i = 0; i < 4; ++i) mfma_tile(fb, i, s1, full);
        epilogue_l2(nch2 - 1);
    };
    if (nrt == 4)
        stream(std::true_type{});
    else
        stream(std::false_type{});
    wait_all_loads();
}

}  // namespace

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_l1(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t st2[kStageBytes];
    __shared__ float s_w[2][kBM];
    __shared__ MTile s_tiles[kTileCache];
    __shared__ int32_t s_tok[kBM];
    gemm_persistent<kL1>(args, st0, st1, st2, s_w[0], s_w[1], s_tiles, s_tok);
}

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_l2(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t st0[kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t st1[kStageBytes];
    __shared__ __attribute__((aligned(16))) uint8_t st2[kStageBytes];
    __shared__ MTile s_tiles[kTileCache];
    gemm_persistent<kL2>(args, st0, st1, st2, nullptr, nullptr, s_tiles, nullptr);
}


__global__ __launch_bounds__(kGemmThreads, kDecWorkgroupsPerCU) void k_gemm_l1_decode(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t st[dec_stages(1) * dec_stage_bytes(1)];
    __shared__ float s_w[dec_rows(1)];
    gemm_decode<kL1, 1>(args, st, s_w);
}

__global__ __launch_bounds__(kGemmThreads, kDecWorkgroupsPerCU) void k_gemm_l1_decode_nt(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t st[dec_stages(1) * dec_stage_bytes(1)];
    __shared__ float s_w[dec_rows(1)];
    gemm_decode<kL1, 1, true>(args, st, s_w);
}

__global__ __launch_bounds__(kGemmThreads, kDecWorkgroupsPerCU) void k_gemm_l2_decode(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t st[dec_stages(1) * dec_stage_bytes(1)];
    gemm_decode<kL2, 1>(args, st, nullptr);
}

__global__ __launch_bounds__(kGemmThreads, kDecWorkgroupsPerCU) void k_gemm_l1_t128(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t st[dec_stages(2) * dec_stage_bytes(2)];
    __shared__ float s_w[dec_rows(2)];
    gemm_decode<kL1, 2>(args, st, s_w);
}

__global__ __launch_bounds__(kGemmThreads, kDecWorkgroupsPerCU) void k_gemm_l2_t128(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t st[dec_stages(2) * dec_stage_bytes(2)];
    gemm_decode<kL2, 2>(args, st, nullptr);
}

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_fused(GemmArgs l1, GemmArgs l2) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kFusedLds];
    gemm_fused(l1, l2, lds);
}

// One 16-byte chunk per thread, in the order of the tile-blocked layout
// (consecutive threads write consecutive chunks): block (e, nt, k) holds
// rows r = 0..255 of 64 bytes, row r being weight row 256 nt + r (L2) or
// gate row 128 nt + r / up row I + 128 nt + r - 128 (L1).
__global__ __launch_bounds__(256) void k_pack_weights_tiled(const uint8_t* __restrict__ W,
                                                           uint8_t* __restrict__ Wp, int E, int N,
                                                           int Kdim, int I, int l1) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int nk = Kdim / kBK, ntiles = N / kBN;
    const int64_t total = (int64_t)E * N * (Kdim / 2) / 16;
    if (q >= total) return;
    const int64_t blk = q >> 10;  // 1024 chunks per block
    const int rem = (int)(q & 1023), r = rem >> 2, ch = rem & 3;
    const int k = (int)(blk % nk);
    const int64_t t = blk / nk;
    const int nt = (int)(t % ntiles), e = (int)(t / ntiles);
    const int w = l1 ? (r < 128 ? 0 : I) + 128 * nt + (r & 127) : kBN * nt + r;
    const uint4 v = *reinterpret_cast<const uint4*>(W + ((int64_t)e * N + w) * (Kdim / 2) + k * (kBK / 2) + 16 * ch);
    *reinterpret_cast<uint4*>(Wp + q * 16) = v;
}

}  // namespace moe
