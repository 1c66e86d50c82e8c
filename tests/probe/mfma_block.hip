// mfma_block.hip -- test infrastructure: one scaled MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, A = e4m3, B = e2m1, one UE8M0 scale per
// 32 along K on each operand) per 32 x 32 x 64 block, with a zero
// accumulator, so that a test can compare each block's result with the exact
// sum of its products; also the MFMA-rate and HBM read-rate probes.  Not part
// of the layer library.
//
// Operand lane layout (the same one the layer's GEMMs use):
//  A (8 VGPRs): lane l holds row l%32; bytes 0-15 are k = 16*(l/32)+0..15,
//    bytes 16-31 are k = 32 + 16*(l/32) + 0..15.
//  B (4 VGPRs of 8): lane l holds column l%32, k = 32*(l/32) + 0..31, two
//    codes per byte, even k in the low nibble.
//  Scales: lane l gives the scale of row (column) l%32 for k-block l/32,
//    byte 0 of its scale register.
//  D (16 fp32): lane l, register r is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Block b: A [32 rows][64 k] e4m3 codes, B [32 columns][32 bytes] (64 e2m1
// codes per column), sa [32 rows][2 k-blocks], sb [32 columns][2 k-blocks],
// D [32 rows][32 columns] fp32.  One 64-lane workgroup per block.
__global__ __launch_bounds__(64) void k_mfma_block(const uint8_t* __restrict__ A,
                                                   const uint8_t* __restrict__ B,
                                                   const uint8_t* __restrict__ sa,
                                                   const uint8_t* __restrict__ sb,
                                                   float* __restrict__ D) {
    const int b = blockIdx.x, l = threadIdx.x;
    const int row = l & 31, h = l >> 5;
    const uint8_t* a = A + (size_t)b * 32 * 64 + row * 64;
    const uint8_t* bb = B + (size_t)b * 32 * 32 + row * 32 + 16 * h;  // column l%32
    v8i av, bv;
    for (int d = 0; d < 4; ++d) {
        int w0 = 0, w1 = 0;
        for (int j = 0; j < 4; ++j) {
            w0 |= (int)a[16 * h + 4 * d + j] << (8 * j);
            w1 |= (int)a[32 + 16 * h + 4 * d + j] << (8 * j);
        }
        av[d] = w0;
        av[4 + d] = w1;
        int wb = 0;
        for (int j = 0; j < 4; ++j) wb |= (int)bb[4 * d + j] << (8 * j);
        bv[d] = wb;
        bv[4 + d] = 0;
    }
    const int sA = sa[(size_t)b * 64 + row * 2 + h];
    const int sB = sb[(size_t)b * 64 + row * 2 + h];
    v16f c;
    for (int r = 0; r < 16; ++r) c[r] = 0.f;
    c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 0, 4, 0, sA, 0, sB);
    for (int r = 0; r < 16; ++r) {
        const int orow = 8 * (r >> 2) + 4 * h + (r & 3);
        D[(size_t)b * 1024 + orow * 32 + row] = c[r];
    }
}

extern "C" int mfma_block_run(const void* A, const void* B, const void* sa, const void* sb,
                              void* D, int nblocks, void* stream) {
    if (nblocks < 1 || !A || !B || !sa || !sb || !D) return -1;
    hipLaunchKernelGGL(k_mfma_block, dim3(nblocks), dim3(64), 0, (hipStream_t)stream,
                       (const uint8_t*)A, (const uint8_t*)B, (const uint8_t*)sa,
                       (const uint8_t*)sb, (float*)D);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

// ---- throughput of the same MFMA with register-resident operands ----------
// Every wave runs `iters` rounds of 8 independent accumulator chains
// (v_mfma_scale_f32_32x32x64_f8f6f4, A format 0 = e4m3, B format fmt_b: 4 =
// e2m1, 0 = e4m3), no memory traffic in the loop.  Operands: `random` = 0 ->
// one constant byte pattern in every operand; 1 -> four pseudo-random operand
// sets per lane, rotated between MFMAs so consecutive MFMAs see different
// bits (as real data does).  One 256-thread workgroup per CU; out gets a
// checksum so the loop is kept.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16; x *= 0x7feb352dU; x ^= x >> 15; x *= 0x846ca68bU; x ^= x >> 16;
    return x;
}

template <int FMT_B>
__device__ __forceinline__ void mfma_rate_body(int iters, int random, float* out) {
    const uint32_t lane = threadIdx.x + 256u * blockIdx.x;
    v8i a[4], b[4];
    for (int s = 0; s < 4; ++s)
        for (int r = 0; r < 8; ++r) {
            const uint32_t ra = random ? mix32(lane * 64u + 16u * s + r) : 0x3C3C3C3Cu;
            const uint32_t rb = random ? mix32(0x9e3779b9u ^ (lane * 64u + 16u * s + r)) : 0x3C3C3C3Cu;
            // e4m3: avoid the NaN codes 0x7F / 0xFF
            a[s][r] = (int)(ra & 0xF7F7F7F7u);
            b[s][r] = (int)(FMT_B == 0 ? (rb & 0xF7F7F7F7u) : rb);
            if (FMT_B == 4 && r >= 4) b[s][r] = 0;  // e2m1 uses 4 registers
        }
    v16f acc[8];
    for (int j = 0; j < 8; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    // rounds in groups of 4 so every operand index is a compile-time constant
    for (int it = 0; it < iters; it += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j & 3], b[(j + u) & 3], acc[j], 0,
                                                                          FMT_B, 0, 127, 0, 127);
    }
    float s = 0.f;
    for (int j = 0; j < 8; ++j)
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[lane] = s;
}

__global__ __launch_bounds__(256, 1) void k_mfma_rate_fp4(int iters, int random, float* out) {
    mfma_rate_body<4>(iters, random, out);
}
__global__ __launch_bounds__(256, 1) void k_mfma_rate_fp8(int iters, int random, float* out) {
    mfma_rate_body<0>(iters, random, out);
}

// Runs the loop (iters rounded up to a multiple of 4) on `blocks` workgroups; B format 4 (e2m1) or 0 (e4m3).
// Returns the elapsed milliseconds from HIP events (or a negative value on
// a failed launch).  out must hold blocks * 256 floats.
extern "C" float mfma_rate_run(int fmt_b, int random, int iters, int blocks, void* out) {
    if (blocks < 1 || iters < 1 || !out || (fmt_b != 0 && fmt_b != 4)) return -1.f;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -2.f;
    hipEventRecord(e0, nullptr);
    if (fmt_b == 4)
        hipLaunchKernelGGL(k_mfma_rate_fp4, dim3(blocks), dim3(256), 0, nullptr, iters, random, (float*)out);
    else
        hipLaunchKernelGGL(k_mfma_rate_fp8, dim3(blocks), dim3(256), 0, nullptr, iters, random, (float*)out);
    hipEventRecord(e1, nullptr);
    float ms = -3.f;
    if (hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess)
        hipEventElapsedTime(&ms, e0, e1);
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    return ms;
}

// ---------------------------------------------------------------------------
// HBM read-stream rate: each workgroup reads one contiguous span of a buffer
// with 16-byte loads, eight per lane in flight, with or without the
// non-temporal hint, and folds the data so the loads stay.  Gives the read
// rate a streaming kernel reaches, beside the 8 TB/s peak.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ __launch_bounds__(256) void k_hbm_read(const u32x4_t* __restrict__ p, size_t n16, size_t per_block,
                                                  unsigned* __restrict__ out) {
    const size_t base = (size_t)blockIdx.x * per_block;
    unsigned acc = 0;
    for (size_t i = base + threadIdx.x; i < base + per_block; i += 256 * 8) {
        u32x4_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t j = i + (size_t)u * 256;
            v[u] = j < n16 ? (NT ? __builtin_nontemporal_load(p + j) : p[j]) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) out[blockIdx.x] = acc;  // practically never: keeps the loads
}

// bytes must be a multiple of 16 * blocks; out holds at least `blocks` words.
extern "C" int hbm_read_run(const void* p, size_t bytes, int blocks, int nt, void* out, void* stream) {
    const size_t n16 = bytes / 16;
    if (blocks <= 0 || bytes % 16 || n16 % (size_t)blocks) return -1;
    const size_t per = n16 / blocks;
    const u32x4_t* P = static_cast<const u32x4_t*>(p);
    unsigned* O = static_cast<unsigned*>(out);
    if (nt)
        hipLaunchKernelGGL(k_hbm_read<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, P, n16, per, O);
    else
        hipLaunchKernelGGL(k_hbm_read<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, P, n16, per, O);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}
