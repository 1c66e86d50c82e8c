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
//  - 256 x 256 tile per 4-wave workgroup, each wave 128 x 128 (4 x 4 MFMA
//    tiles); K steps of 128; global -> VGPR prefetch two steps ahead,
//    VGPR -> LDS double buffer, XOR-swizzled 16-byte chunks so that the MFMA
//    fragment reads are bank-conflict free.
//  - Expert-major m-tile table built on the device by the routing scan: no
//    host synchronisation; surplus workgroups exit at once.
//  - Workgroup ids are remapped so that each XCD (own L2) works on a
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

// Which expert-matrix row (output column) holds LDS B row `nrow` of tile nt.
template <int MODE>
__device__ __forceinline__ int b_row(int nt, int nrow, int I) {
    if (MODE == kL1) {
        // rows 0..127: gate columns nt*128 + nrow; 128..255: the matching up columns
        return nrow < 128 ? nt * 128 + nrow : I + nt * 128 + (nrow - 128);
    }
    return nt * kBN + nrow;
}

// LDS B row of this wave's column tile j (0..3).
template <int MODE>
__device__ __forceinline__ int wave_b_row0(int wn, int j) {
    if (MODE == kL1) return (j < 2 ? 0 : 128) + 64 * wn + 32 * (j & 1);
    return 128 * wn + 32 * j;
}

__device__ __forceinline__ int tile_of_block(int bid, int nblk) {
    // Hardware hands out workgroups round-robin over 8 XCDs; give XCD x a
    // contiguous range of logical tiles instead.
    const int per = nblk / 8, rem = nblk % 8;
    const int xcd = bid % 8, j = bid / 8;
    return xcd * per + min(xcd, rem) + j;
}

struct Frags {
    v8i a[4];
    v8i b[4];
    int sa[4];
    int sb[4];
};

template <int MODE>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, uint8_t* smem) {
    const int tid = threadIdx.x;
    const int wid = tid / 64, lane = tid % 64;
    const int wm = wid >> 1, wn = wid & 1;
    const int h = lane >> 5, l32 = lane & 31;

    const int logical = tile_of_block(blockIdx.x, gridDim.x);
    const int mt = logical / g.ntiles, nt = logical % g.ntiles;
    if (mt >= *g.num_mtiles) return;
    const MTile tile = g.mtiles[mt];
    const int e = tile.expert, row0 = tile.row0, nrows = tile.nrows;
    const int Kdim = g.Kdim;
    const int nk = Kdim / kBK;

    float* s_w = reinterpret_cast<float*>(smem + kStages * kStageBytes);
    if (MODE == kL1) s_w[tid] = tid < nrows ? g.pool_w[row0 + tid] : 0.f;

    // ---- global -> register staging addresses (constant per thread) -------
    // A: 2048 16-byte chunks per step; chunk q = tid + 256 i covers LDS row
    // q/8, physical chunk q%8, holding logical chunk (q%8) ^ (row%8).
    const int a_row = tid >> 3;                     // + 32 i
    const int a_chunk = (tid & 7) ^ ((tid >> 3) & 7);
    const uint8_t* a_src = g.A + (int64_t)(row0 + a_row) * Kdim + 16 * a_chunk;
    const int64_t a_stride32 = (int64_t)32 * Kdim;
    // B: 1024 chunks; chunk q = tid + 256 i covers LDS row q/4, physical
    // chunk q%4, logical chunk (q%4) ^ ((row/2)%4).
    const int b_chunk = (tid & 3) ^ ((tid >> 3) & 3);
    const int64_t b_ld = Kdim / 2;
    const uint8_t* b_exp = g.B + (int64_t)e * g.N * b_ld + 16 * b_chunk;
    const uint8_t* b_src0 = b_exp + b_row<MODE>(nt, (tid >> 2), g.I) * b_ld;
    const uint8_t* b_src1 = b_exp + b_row<MODE>(nt, (tid >> 2) + 64, g.I) * b_ld;
    const uint8_t* b_src2 = b_exp + b_row<MODE>(nt, (tid >> 2) + 128, g.I) * b_ld;
    const uint8_t* b_src3 = b_exp + b_row<MODE>(nt, (tid >> 2) + 192, g.I) * b_ld;
    // scales: one dword (4 k-blocks) per row per step
    const uint8_t* sa_src = g.SA + (int64_t)(row0 + tid) * (Kdim / 32);
    const uint8_t* sb_src = g.SB + ((int64_t)e * g.N + b_row<MODE>(nt, tid, g.I)) * (Kdim / 32);

    // Staging registers as named scalars (arrays of them would be moved to
    // LDS by the compiler's alloca promotion).
    uint4 ra0, ra1, ra2, ra3, ra4, ra5, ra6, ra7, rb0, rb1, rb2, rb3;
    uint32_t rsa, rsb;
    auto load_global = [&](int kk) __attribute__((always_inline)) {
        const int k0 = kk * kBK;
        const uint8_t* pa = a_src + k0;
        ra0 = *reinterpret_cast<const uint4*>(pa);
        ra1 = *reinterpret_cast<const uint4*>(pa + a_stride32);
        ra2 = *reinterpret_cast<const uint4*>(pa + 2 * a_stride32);
        ra3 = *reinterpret_cast<const uint4*>(pa + 3 * a_stride32);
        ra4 = *reinterpret_cast<const uint4*>(pa + 4 * a_stride32);
        ra5 = *reinterpret_cast<const uint4*>(pa + 5 * a_stride32);
        ra6 = *reinterpret_cast<const uint4*>(pa + 6 * a_stride32);
        ra7 = *reinterpret_cast<const uint4*>(pa + 7 * a_stride32);
        rb0 = *reinterpret_cast<const uint4*>(b_src0 + k0 / 2);
        rb1 = *reinterpret_cast<const uint4*>(b_src1 + k0 / 2);
        rb2 = *reinterpret_cast<const uint4*>(b_src2 + k0 / 2);
        rb3 = *reinterpret_cast<const uint4*>(b_src3 + k0 / 2);
        rsa = *reinterpret_cast<const uint32_t*>(sa_src + k0 / 32);
        rsb = *reinterpret_cast<const uint32_t*>(sb_src + k0 / 32);
    };
    auto store_lds = [&](int st) __attribute__((always_inline)) {
        uint4* pa = reinterpret_cast<uint4*>(smem + st * kStageBytes) + tid;
        pa[0] = ra0;
        pa[256] = ra1;
        pa[512] = ra2;
        pa[768] = ra3;
        pa[1024] = ra4;
        pa[1280] = ra5;
        pa[1536] = ra6;
        pa[1792] = ra7;
        uint4* pb = reinterpret_cast<uint4*>(smem + st * kStageBytes + kStageA) + tid;
        pb[0] = rb0;
        pb[256] = rb1;
        pb[512] = rb2;
        pb[768] = rb3;
        uint32_t* ps = reinterpret_cast<uint32_t*>(smem + st * kStageBytes + kStageA + kStageB) + tid;
        ps[0] = rsa;
        ps[kStageSA / 4] = rsb;
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // ---- fragment read addresses (LDS byte offsets inside a stage) ---------
    // A row of row-tile i: 128*wm + 32*i + l32; row%8 == lane%8.
    const int a_frag_row = 128 * wm + l32;
    const int a_sw = lane & 7;
    // B row of column tile j: wave_b_row0(j) + l32; (row/2)%4 == (l32/2)%4.
    const int b_sw = (l32 >> 1) & 3;

    auto compute = [&](int st) __attribute__((always_inline)) {
        const uint8_t* base = smem + st * kStageBytes;
        const uint8_t* sA = base;
        const uint8_t* sB = base + kStageA;
        const uint32_t* sSA = reinterpret_cast<const uint32_t*>(base + kStageA + kStageB);
        const uint32_t* sSB = reinterpret_cast<const uint32_t*>(base + kStageA + kStageB + kStageSA);
        uint32_t wa[4], wb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) wa[i] = sSA[a_frag_row + 32 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) wb[j] = sSB[wave_b_row0<MODE>(wn, j) + l32];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            Frags f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint8_t* rowp = sA + (a_frag_row + 32 * i) * kBK;
                const uint4 lo = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * s + h) ^ a_sw));
                const uint4 hi = *reinterpret_cast<const uint4*>(rowp + 16 * ((4 * s + 2 + h) ^ a_sw));
                f.a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                             (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                f.sa[i] = (int)(wa[i] >> (8 * (2 * s + h)));
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint8_t* rowp = sB + (wave_b_row0<MODE>(wn, j) + l32) * (kBK / 2);
                const uint4 v = *reinterpret_cast<const uint4*>(rowp + 16 * ((2 * s + h) ^ b_sw));
                f.b[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
                f.sb[j] = (int)(wb[j] >> (8 * (2 * s + h)));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        f.a[i], f.b[j], acc[i][j], 0, 4, 0, f.sa[i], 0, f.sb[j]);
        }
    };

    // ---- main loop: prefetch two steps ahead, two LDS stages ---------------
    load_global(0);
    store_lds(0);
    if (nk > 1) load_global(1);
    __syncthreads();
    for (int kk = 0; kk < nk; ++kk) {
        if (kk + 1 < nk) store_lds((kk + 1) & 1);
        if (kk + 2 < nk) load_global(kk + 2);
        compute(kk & 1);
        __syncthreads();
    }

    // ---- epilogue ------------------------------------------------------------
    uint8_t* wbuf = smem + wid * 8192;  // per-wave staging, stages are free now
    if (MODE == kL2) {
        const int N = g.N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // bf16 tile of 32 rows x 128 columns, row-major, 256 B per row
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
                    const float v = acc[i][j][r];
                    reinterpret_cast<uint16_t*>(wbuf)[rr * 128 + 32 * j + l32] =
                        (uint16_t)pack_bf16x2(v, 0.f);
                }
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const int q = lane + 64 * m;
                const int rr = q >> 4, cu = q & 15;
                const int lrow = 128 * wm + 32 * i + rr;
                const uint4 v = reinterpret_cast<const uint4*>(wbuf)[q];
                if (lrow < nrows)
                    *reinterpret_cast<uint4*>(g.out + (int64_t)(row0 + lrow) * N + nt * kBN +
                                              128 * wn + 8 * cu) = v;
            }
        }
    } else {
        const int I = g.I;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = 8 * (r >> 2) + 4 * h + (r & 3);
                    const int lrow = 128 * wm + 32 * i + rr;
                    const float gt = round_bf16(acc[i][jj][r]);
                    const float up = round_bf16(acc[i][jj + 2][r]);
                    float sl;
                    if (g.fast_math) {
                        const float ex = __builtin_amdgcn_exp2f(-gt * 1.4426950408889634f);
                        sl = gt * __builtin_amdgcn_rcpf(1.0f + ex);
                    } else {
                        sl = gt / (1.0f + expf(-gt));
                    }
                    const float a = (sl * up) * s_w[lrow];
                    const float amax = half_wave_max(fabsf(a));
                    const uint32_t b = ue8m0_e4m3(amax);
                    const uint32_t code = pack_fp8x2(unscale(a, b), 0.f) & 0xFFu;
                    wbuf[rr * 64 + 32 * jj + l32] = (uint8_t)code;
                    if (l32 == 0 && lrow < nrows)
                        g.act_s[(int64_t)(row0 + lrow) * (I / 32) + (nt * 128 + 64 * wn) / 32 + jj] =
                            (uint8_t)b;
                }
            }
            // 32 rows x 64 code bytes -> global, 16 bytes per lane
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int q = lane + 64 * m;
                const int rr = q >> 2, cu = q & 3;
                const int lrow = 128 * wm + 32 * i + rr;
                const uint4 v = reinterpret_cast<const uint4*>(wbuf)[q];
                if (lrow < nrows)
                    *reinterpret_cast<uint4*>(g.act_q + (int64_t)(row0 + lrow) * I + nt * 128 +
                                              64 * wn + 16 * cu) = v;
            }
        }
    }
}

}  // namespace

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_l1(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kGemmLds];
    gemm_tile<kL1>(args, smem);
}

__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm_l2(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[kGemmLds];
    gemm_tile<kL2>(args, smem);
}

}  // namespace moe
