// route.hip -- dispatch (a1-a4) and combine (a9) kernels for gfx950.
//
// Dispatch follows the counting-sort shape the pages describe for the
// dispatch warps (page "Dispatch/Combine in Mega MoE", sections 3.1 and 8.3;
// page "DeepEP -> Mega MoE", "dispatch.cuh" snippets): a per-expert count of
// topk_idx, an exclusive prefix sum into per-expert offsets, a slot inside the
// expert, then a copy of the token row into that expert-major pool slot.
// Differences from the pages' design, for one GPU and a deterministic result:
//  - slots are ranked stably (ascending flat slot t*K+k inside an expert)
//    instead of by atomic arrival order;
//  - the histogram is privatised per wave in LDS over fixed kSegSlots-slot
//    segments, so the ranking pass can start each segment from an exact base;
//  - the token row is quantised to e4m3 while it is copied (the pages pull
//    rows that are already FP8; quantising per row before or after the copy
//    gives the same bytes).
#include "moe_device.hpp"
#include "moe_kernels.hpp"

namespace moe {

// a1: per-segment expert histogram.  One wave per kSegSlots-slot segment, LDS
// atomics on a per-wave histogram.  Indices >= E are counted as errors and
// otherwise treated as masked.
__device__ __forceinline__ void route_count_block(const int64_t* __restrict__ topk_idx, int64_t TK,
                                                  int E, int32_t* __restrict__ seg_hist,
                                                  int32_t* __restrict__ seg_err, int64_t blk,
                                                  int32_t* lds_hist /* [kRouteWaves][E] */,
                                                  int32_t* __restrict__ blk_hist = nullptr,
                                                  int32_t* __restrict__ blk_err = nullptr) {
    const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t nseg = (TK + kSegSlots - 1) / kSegSlots;
    const int64_t seg = blk * kRouteWaves + wv;
    int32_t* h = lds_hist + wv * E;
    for (int e = lane; e < E; e += kWave) h[e] = 0;
    __syncthreads();
    int bad = 0;
    if (seg < nseg) {
        const int64_t f0 = seg * kSegSlots;
        for (int i = lane; i < kSegSlots; i += kWave) {
            const int64_t f = f0 + i;
            if (f >= TK) break;
            const int64_t e = topk_idx[f];
            if (e >= E)
                bad = 1;
            else if (e >= 0)
                atomicAdd(&h[e], 1);
        }
    }
    __syncthreads();
    if (blk_hist) {
        // the block's four segments summed: one histogram row per block
        __shared__ int32_t s_bad;
        if (threadIdx.x == 0) s_bad = 0;
        __syncthreads();
        if (bad) s_bad = 1;
        for (int e = threadIdx.x; e < E; e += kRouteThreads) {
            int sum = 0;
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) sum += lds_hist[w * E + e];
            blk_hist[blk * E + e] = sum;
        }
        __syncthreads();
        if (threadIdx.x == 0) blk_err[blk] = s_bad;
        return;
    }
    if (seg < nseg) {
        for (int e = lane; e < E; e += kWave) seg_hist[seg * E + e] = h[e];
        const unsigned long long any_bad = __ballot(bad);
        if (lane == 0) seg_err[seg] = any_bad ? 1 : 0;
    }
}

__global__ __launch_bounds__(kRouteThreads) void k_route_count(
    const int64_t* __restrict__ topk_idx, int64_t TK, int E, int32_t* __restrict__ seg_hist,
    int32_t* __restrict__ seg_err, int32_t* __restrict__ blk_hist, int32_t* __restrict__ blk_err) {
    extern __shared__ int32_t lds_hist[];  // [kRouteWaves][E]
    route_count_block(topk_idx, TK, E, seg_hist, seg_err, blockIdx.x, lds_hist, blk_hist, blk_err);
}

// a2: exclusive prefix sum.  One block.  The segment histogram [nseg][E] is
// split among P threads per expert (P a power of two, P*E <= blockDim;
// thread tid = p*E + e, so a wave reads consecutive experts of a segment):
// each sums its chunk of segments, the chunk sums are scanned per expert,
// then a block-wide scan over experts gives offsets[E+1] and, over
// ceil(count/kBM), the GEMM's expert-major m-tile table; finally each thread
// walks its chunk again writing the per-segment bases.
__global__ __launch_bounds__(1024) void k_route_scan(
    const int32_t* __restrict__ seg_hist, const int32_t* __restrict__ seg_err, int nseg, int E,
    int32_t* __restrict__ seg_base, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    MTile* __restrict__ mtiles, int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag) {
    __shared__ int32_t s_part[1024];  // chunk sums, then chunk bases inside the expert
    __shared__ int32_t s_cnt[1024];   // count per expert, then offset per expert
    __shared__ int32_t wsum[16], wsum_t[16], werr[16];
    const int tid = threadIdx.x;
    int P = 1;
    while (2 * P * E <= (int)blockDim.x) P *= 2;
    const int e_of = tid % E, p_of = tid / E;
    const bool owner = p_of < P;  // tid < P*E
    const int C = (nseg + P - 1) / P;
    const int s0 = min(nseg, p_of * C), s1 = min(nseg, s0 + C);
    if (owner) {
        int sum = 0;
#pragma unroll 8
        for (int sg = s0; sg < s1; ++sg) sum += seg_hist[(int64_t)sg * E + e_of];
        s_part[tid] = sum;
    }
    int err = 0;
    for (int sg = tid; sg < nseg; sg += blockDim.x) err |= seg_err[sg];
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int q = 0; q < P; ++q) {
            const int v = s_part[q * E + tid];
            s_part[q * E + tid] = run;
            run += v;
        }
        s_cnt[tid] = run;
    }
    __syncthreads();

    // scan over experts: thread e (< E) owns expert e
    const int e = tid;
    const int lane = e % kWave, wv = e / kWave;
    const int cnt = e < E ? s_cnt[e] : 0;
    const int nt = (cnt + kBM - 1) / kBM;
    int inc = cnt, inc_t = nt;
    for (int d = 1; d < kWave; d <<= 1) {
        const int a = __shfl_up(inc, d), b = __shfl_up(inc_t, d);
        if (lane >= d) {
            inc += a;
            inc_t += b;
        }
    }
    const unsigned long long eb = __ballot(err);
    if (lane == kWave - 1) {
        wsum[wv] = inc;
        wsum_t[wv] = inc_t;
    }
    if (lane == 0) werr[wv] = eb ? 1 : 0;
    __syncthreads();
    int base = 0, base_t = 0, any_err = 0;
    for (int i = 0; i < (int)(blockDim.x / kWave); ++i) {
        if (i < wv) {
            base += wsum[i];
            base_t += wsum_t[i];
        }
        any_err |= werr[i];
    }
    const int off = base + inc - cnt;
    const int toff = base_t + inc_t - nt;
    if (e < E) {
        counts[e] = cnt;
        offsets[e] = off;
        for (int i = 0; i < nt; ++i) {
            MTile m;
            m.expert = e;
            m.row0 = off + i * kBM;
            m.nrows = min(kBM, cnt - i * kBM);
            m.pad = 0;
            mtiles[toff + i] = m;
        }
    }
    if (e == E - 1) {
        offsets[E] = off + cnt;
        *num_mtiles = toff + nt;
        *err_flag = any_err;
    }
    __syncthreads();  // s_cnt now read as counts by every owner below
    if (e < E) s_cnt[e] = off;
    __syncthreads();
    if (owner) {
        int run = s_cnt[e_of] + s_part[tid];
#pragma unroll 8
        for (int sg = s0; sg < s1; ++sg) {
            const int64_t i = (int64_t)sg * E + e_of;
            const int v = seg_hist[i];
            seg_base[i] = run;
            run += v;
        }
    }
}

// a3: stable rank.  Each wave walks its segment 64 slots at a time; lanes
// holding the same expert find each other with one ballot per index bit, the
// lower lanes go first, and one lane advances the expert's running base in
// LDS.  The segment bases come from k_route_scan, so pool rows come out in
// ascending flat-slot order inside every expert.
__global__ __launch_bounds__(kRouteThreads) void k_route_scatter(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int64_t TK, int E,
    int nbits, int K, const int32_t* __restrict__ seg_base, int32_t* __restrict__ pool_src,
    int32_t* __restrict__ slot_to_pool, float* __restrict__ pool_w, int32_t* __restrict__ pool_tok) {
    extern __shared__ int32_t lds_run[];  // [kRouteWaves][E]
    const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t nseg = (TK + kSegSlots - 1) / kSegSlots;
    const int64_t seg = (int64_t)blockIdx.x * kRouteWaves + wv;
    int32_t* run = lds_run + wv * E;
    if (seg < nseg)
        for (int e = lane; e < E; e += kWave) run[e] = seg_base[seg * E + e];
    __syncthreads();
    if (seg >= nseg) return;
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    const int64_t f0 = seg * kSegSlots;
    for (int it = 0; it < kSegSlots / kWave; ++it) {
        const int64_t f = f0 + it * kWave + lane;
        if (f0 + it * kWave >= TK) break;  // wave-uniform
        int e = -1;
        float w = 0.f;
        if (f < TK) {
            const int64_t v = topk_idx[f];
            if (v >= 0 && v < E) {
                e = (int)v;
                w = topk_w[f];
            }
        }
        unsigned long long peers = __ballot(e >= 0);
        for (int b = 0; b < nbits; ++b) {
            const int bit = (e >> b) & 1;
            const unsigned long long set = __ballot(bit);
            peers &= bit ? set : ~set;
        }
        if (e >= 0) {
            const int base = run[e];
            const int r = base + __popcll(peers & lt_mask);
            pool_src[r] = (int32_t)f;
            slot_to_pool[f] = r;
            pool_w[r] = w;
            if (pool_tok) pool_tok[r] = (int32_t)(f / K);
            if ((peers >> lane) == 1ull) run[e] = base + __popcll(peers);  // highest peer lane
        } else if (f < TK) {
            slot_to_pool[f] = -1;
        }
    }
}

// Block-wide exclusive scan of v over the block's threads (kRouteThreads);
// returns the thread's exclusive prefix and sets *total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int32_t* s_w /* [kRouteWaves] */) {
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    int inc = v;
    for (int d = 1; d < kWave; d <<= 1) {
        const int a = __shfl_up(inc, d);
        if (lane >= d) inc += a;
    }
    __syncthreads();  // s_w free
    if (lane == kWave - 1) s_w[wv] = inc;
    __syncthreads();
    int base = 0, tot = 0;
    for (int i = 0; i < kRouteWaves; ++i) {
        if (i < wv) base += s_w[i];
        tot += s_w[i];
    }
    *total = tot;
    return base + inc - v;
}

// The routing's outputs besides the per-slot ones, written by one block from
// the expert totals s_tot and offsets s_off in its LDS (R rows in all, err
// set if an expert index was >= E): counts, offsets[E+1], the expert-major
// m-tile table (tiles of kBM rows) and, with mtiles64 set, the same rows in
// tiles of dec_rows rows, and the error flag.  Thread tid owns experts
// [ept tid, ept tid + ept); s_w: kRouteWaves words of scan scratch.
__device__ __forceinline__ void route_write_tables(int E, int R, int err, const int32_t* s_tot,
                                                   const int32_t* s_off, int32_t* s_w,
                                                   int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                   MTile* __restrict__ mtiles, int32_t* __restrict__ num_mtiles,
                                                   int32_t* __restrict__ err_flag, MTile* __restrict__ mtiles64,
                                                   int32_t* __restrict__ num_mtiles64, int dec_rows) {
    const int tid = threadIdx.x;
    const int ept = (E + kRouteThreads - 1) / kRouteThreads;
    int my_nt = 0;
    for (int j = 0; j < ept; ++j) {
        const int e = ept * tid + j;
        if (e < E) my_nt += (s_tot[e] + kBM - 1) / kBM;
    }
    int ntot = 0;
    int toff = block_exclusive_scan(my_nt, &ntot, s_w);
    for (int j = 0; j < ept; ++j) {
        const int e = ept * tid + j;
        if (e >= E) continue;
        const int cnt = s_tot[e], nt = (cnt + kBM - 1) / kBM;
        counts[e] = cnt;
        offsets[e] = s_off[e];
        for (int i = 0; i < nt; ++i) {
            MTile m;
            m.expert = e;
            m.row0 = s_off[e] + i * kBM;
            m.nrows = min(kBM, cnt - i * kBM);
            m.pad = 0;
            mtiles[toff + i] = m;
        }
        toff += nt;
    }
    int ntot64 = 0;
    if (mtiles64) {
        int my64 = 0;
        for (int j = 0; j < ept; ++j) {
            const int e = ept * tid + j;
            if (e < E) my64 += (s_tot[e] + dec_rows - 1) / dec_rows;
        }
        int t64 = block_exclusive_scan(my64, &ntot64, s_w);
        for (int j = 0; j < ept; ++j) {
            const int e = ept * tid + j;
            if (e >= E) continue;
            const int cnt = s_tot[e], nt = (cnt + dec_rows - 1) / dec_rows;
            for (int i = 0; i < nt; ++i) {
                MTile m;
                m.expert = e;
                m.row0 = s_off[e] + i * dec_rows;
                m.nrows = min(dec_rows, cnt - i * dec_rows);
                m.pad = 0;
                mtiles64[t64 + i] = m;
            }
            t64 += nt;
        }
    }
    if (tid == 0) {
        offsets[E] = R;
        *num_mtiles = ntot;
        if (num_mtiles64) *num_mtiles64 = ntot64;
        *err_flag = err ? 1 : 0;
    }
}

// a2 + a3 + the pool rows' scale words, in one launch.  Block b takes the
// kRouteWaves segments the counting pass's block b counted (wave w: segment
// kRouteWaves*b + w) and works out for itself what a scan over that pass's
// per-block histograms blk_hist [nblk][E] gives it -- each expert's total
// (hence offsets[E+1]) and its rows in blocks before b -- so that no block
// waits for another.  Then, as in the counting-sort dispatch the pages
// describe: the per-segment base of every expert, the stable rank of every
// valid slot inside its expert (lanes holding the same expert find each
// other with one ballot per index bit; lower lanes first), and the pool row
// of every slot.  With pool_s set, the block then copies the A-scale words of
// its pool rows from their tokens' words (tok_s, [T][W]) into the GEMM's
// packed k-major layout (word (w, r) at w * cap + r), one thread per row in
// the order of the rows.  Block 0 also writes counts, offsets, the GEMM's
// expert-major m-tile table (and with mtiles64 set the same rows in tiles
// of at most dec_rows rows) and the routing error flag.
__device__ __forceinline__ void route_block(
    int b, const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int64_t TK, int E,
    int nbits, int K, const int32_t* __restrict__ blk_hist, const int32_t* __restrict__ blk_err,
    int nblk, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    MTile* __restrict__ mtiles, int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag,
    int32_t* __restrict__ pool_src, int32_t* __restrict__ slot_to_pool, float* __restrict__ pool_w,
    int32_t* __restrict__ pool_tok, const uint32_t* __restrict__ tok_s, int W, int64_t cap,
    uint32_t* __restrict__ pool_s, MTile* __restrict__ mtiles64, int32_t* __restrict__ num_mtiles64,
    int dec_rows, int32_t* lds /* route_lds_bytes(E) */) {
    int32_t* s_tot = lds;                     // [E] expert totals
    int32_t* s_pre = s_tot + E;               // [E] rows of the expert in blocks before this one
    int32_t* s_run = s_pre + E;               // [kRouteWaves][E] per-wave counts, then running bases
    int32_t* s_off = s_run + kRouteWaves * E; // [E] offsets
    int32_t* s_loc = s_off + E;               // [E] first slot of the expert in this block's row list
    int2* s_rows = reinterpret_cast<int2*>(s_loc + E);  // [kRouteWaves * kSegSlots] (row, token)
    __shared__ int32_t s_part[2][kRouteThreads];
    __shared__ int32_t s_w[kRouteWaves];
    __shared__ int32_t s_nrows;
    const int tid = threadIdx.x, wv = tid / kWave, lane = tid % kWave;
    const int64_t nseg = (TK + kSegSlots - 1) / kSegSlots;
    const int64_t seg = (int64_t)b * kRouteWaves + wv;
    const int64_t f0 = seg * kSegSlots;

    // the wave's slots (indices and weights, all loads at once), and this
    // block's own segments counted again (one histogram per wave)
    constexpr int kIt = kSegSlots / kWave;
    int sl_e[kIt];
    float sl_w[kIt];
#pragma unroll
    for (int it = 0; it < kIt; ++it) {
        const int64_t f = f0 + it * kWave + lane;
        sl_e[it] = -1;
        sl_w[it] = 0.f;
        if (seg < nseg && f < TK) {
            const int64_t v = topk_idx[f];
            if (v >= 0 && v < E) {
                sl_e[it] = (int)v;
                sl_w[it] = topk_w[f];
            }
        }
    }
    int32_t* h = s_run + wv * E;
    for (int e = lane; e < E; e += kWave) h[e] = 0;
    __syncthreads();
#pragma unroll
    for (int it = 0; it < kIt; ++it)
        if (sl_e[it] >= 0) atomicAdd(&h[sl_e[it]], 1);

    // expert totals and rows in earlier blocks: P threads per expert, each
    // summing a run of the blocks' histograms
    int P = 1;
    while (2 * P * E <= kRouteThreads) P *= 2;
    for (int x = tid; x < P * E; x += kRouteThreads) {
        const int e = x % E, p = x / E;
        const int C = (nblk + P - 1) / P;
        const int b0 = min(nblk, p * C), b1 = min(nblk, b0 + C);
        int tot = 0, pre = 0;
#pragma unroll 8
        for (int bb = b0; bb < b1; ++bb) {
            const int v = blk_hist[(int64_t)bb * E + e];
            tot += v;
            pre += bb < b ? v : 0;
        }
        if (P == 1) {
            s_tot[e] = tot;
            s_pre[e] = pre;
        } else {
            s_part[0][x] = tot;
            s_part[1][x] = pre;
        }
    }
    __syncthreads();
    if (P > 1)
        for (int e = tid; e < E; e += kRouteThreads) {
            int tot = 0, pre = 0;
            for (int p = 0; p < P; ++p) {
                tot += s_part[0][p * E + e];
                pre += s_part[1][p * E + e];
            }
            s_tot[e] = tot;
            s_pre[e] = pre;
        }
    __syncthreads();

    // offsets (exclusive scan of the totals) and each expert's first slot in
    // this block's row list (exclusive scan of the block's counts); thread
    // tid owns experts [ept*tid, ept*tid + ept)
    const int ept = (E + kRouteThreads - 1) / kRouteThreads;
    int my_tot = 0, my_blk = 0;
    for (int j = 0; j < ept; ++j) {
        const int e = ept * tid + j;
        if (e < E) {
            my_tot += s_tot[e];
            int c = 0;
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) c += s_run[w * E + e];
            my_blk += c;
        }
    }
    int R = 0, nrows = 0;
    int off = block_exclusive_scan(my_tot, &R, s_w);
    int loc = block_exclusive_scan(my_blk, &nrows, s_w);
    for (int j = 0; j < ept; ++j) {
        const int e = ept * tid + j;
        if (e < E) {
            s_off[e] = off;
            s_loc[e] = loc;
            // running bases of the block's waves: the expert's offset, its rows
            // in earlier blocks, then the earlier waves of this block
            int run = off + s_pre[e];
#pragma unroll
            for (int w = 0; w < kRouteWaves; ++w) {
                const int c = s_run[w * E + e];
                s_run[w * E + e] = run;
                run += c;
            }
            off += s_tot[e];
            loc += run - (s_off[e] + s_pre[e]);  // the block's rows of expert e
        }
    }
    if (tid == 0) s_nrows = nrows;
    __syncthreads();

    // the stable rank of every slot of the wave's segment
    if (seg < nseg) {
        int32_t* run = s_run + wv * E;
        const unsigned long long lt_mask = (1ull << lane) - 1ull;
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int64_t f = f0 + it * kWave + lane;
            if (f0 + it * kWave >= TK) break;  // wave-uniform
            const int e = sl_e[it];
            const float w = sl_w[it];
            unsigned long long peers = __ballot(e >= 0);
            for (int bt = 0; bt < nbits; ++bt) {
                const int bit = (e >> bt) & 1;
                const unsigned long long set = __ballot(bit);
                peers &= bit ? set : ~set;
            }
            if (e >= 0) {
                const int base = run[e];
                const int r = base + __popcll(peers & lt_mask);
                const int32_t t = (int32_t)(f / K);
                pool_src[r] = (int32_t)f;
                slot_to_pool[f] = r;
                pool_w[r] = w;
                if (pool_tok) pool_tok[r] = t;
                // the row's place in the block's list: the block's rows of
                // expert e are the pool rows [s_off + s_pre, ...) in order
                s_rows[s_loc[e] + (r - s_off[e] - s_pre[e])] = make_int2(r, t);
                if ((peers >> lane) == 1ull) run[e] = base + __popcll(peers);  // highest peer lane
            } else if (f < TK) {
                slot_to_pool[f] = -1;
            }
        }
    }
    __syncthreads();

    // the A-scale words of the block's pool rows, rows in ascending order
    // within each expert (consecutive threads write consecutive words)
    if (pool_s) {
        const int n = s_nrows;
        for (int i = tid; i < n; i += kRouteThreads) {
            const int2 rt = s_rows[i];
            const int64_t r = rt.x, t = rt.y;
            if ((W & 3) == 0) {
                const uint4* src = reinterpret_cast<const uint4*>(tok_s + t * W);
                for (int w4 = 0; w4 < W / 4; ++w4) {
                    const uint4 v = src[w4];
                    pool_s[(int64_t)(4 * w4 + 0) * cap + r] = v.x;
                    pool_s[(int64_t)(4 * w4 + 1) * cap + r] = v.y;
                    pool_s[(int64_t)(4 * w4 + 2) * cap + r] = v.z;
                    pool_s[(int64_t)(4 * w4 + 3) * cap + r] = v.w;
                }
            } else {
                for (int w = 0; w < W; ++w) pool_s[(int64_t)w * cap + r] = tok_s[t * W + w];
            }
        }
    }

    if (b == 0) {
        int err = 0;
        for (int bb = tid; bb < nblk; bb += kRouteThreads) err |= blk_err[bb];
        err = __syncthreads_or(err);
        route_write_tables(E, R, err, s_tot, s_off, s_w, counts, offsets, mtiles, num_mtiles, err_flag,
                           mtiles64, num_mtiles64, dec_rows);
    }
}

__global__ __launch_bounds__(kRouteThreads) void k_route(
    const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int64_t TK, int E,
    int nbits, int K, const int32_t* __restrict__ blk_hist, const int32_t* __restrict__ blk_err,
    int nblk, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    MTile* __restrict__ mtiles, int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag,
    int32_t* __restrict__ pool_src, int32_t* __restrict__ slot_to_pool, float* __restrict__ pool_w,
    int32_t* __restrict__ pool_tok, const uint32_t* __restrict__ tok_s, int W, int64_t cap,
    uint32_t* __restrict__ pool_s, MTile* __restrict__ mtiles64, int32_t* __restrict__ num_mtiles64,
    int dec_rows) {
    extern __shared__ int32_t lds[];
    route_block(blockIdx.x, topk_idx, topk_w, TK, E, nbits, K, blk_hist, blk_err, nblk, counts,
                       offsets, mtiles, num_mtiles, err_flag, pool_src, slot_to_pool, pool_w, pool_tok,
                       tok_s, W, cap, pool_s, mtiles64, num_mtiles64, dec_rows, lds);
}

// a4: gather + quantise.  A block takes tpb consecutive token rows (as many
// as fit 8192 columns, else one) as one flat span; each lane owns 8
// consecutive columns of up to four 2048-column chunks, whose 16-byte loads
// all go out first.  A quad of lanes owns one 32-column scale group: amax
// over the quad, UE8M0 scale, e4m3 codes, then the 8 code bytes go to every
// valid pool row of the token -- or, with a null slot_to_pool, once to row t
// of a token-major copy (the fused layer's L1 reads token rows from it
// directly).  The scale bytes go either to every pool row of the token
// (pool_s, [rows][H/32]) or once to the token (tok_s, [T][H/128] words
// holding groups 4w, 4w+2, 4w+1, 4w+3 in byte order, the word form the GEMM
// loads); a null pointer skips that form.
__device__ __forceinline__ void dispatch_fp8_block(const uint16_t* __restrict__ x, int64_t T,
                                                   int H, int K, int tpb,
                                                   const int32_t* __restrict__ slot_to_pool,
                                                   uint8_t* __restrict__ pool,
                                                   uint8_t* __restrict__ pool_s,
                                                   uint8_t* __restrict__ tok_s, int64_t blk) {
    __shared__ int32_t rows[kMaxBlockTokens * 64];
    const int64_t t0 = blk * tpb;
    if (!slot_to_pool) K = 1;  // token-major only: row t of pool is token t
    for (int i = threadIdx.x; i < tpb * K; i += 256) {
        const int64_t t = t0 + i / K;
        rows[i] = t >= T ? -1 : (slot_to_pool ? slot_to_pool[t0 * K + i] : (int32_t)t);
    }
    __syncthreads();
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    // the block's tokens as one flat span; H % 32 == 0, so a quad's 32
    // columns (one scale group) belong to one token
    const int span = tpb * H;
    for (int c00 = threadIdx.x * 8; c00 < span; c00 += 4 * 256 * 8) {
        int tok[4], col[4];
        u32x4 v[4];
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            const int p = c00 + hh * 256 * 8;
            const int j = p < span ? p / H : -1;
            tok[hh] = (j >= 0 && t0 + j < T) ? j : -1;
            col[hh] = j >= 0 ? p - j * H : 0;
            const u32x4 z = {0, 0, 0, 0};
            // streamed: each x byte is read once
            v[hh] = tok[hh] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                       x + (t0 + tok[hh]) * H + col[hh]))
                                 : z;
        }
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            float f[8] = {bf16_lo(v[hh].x), bf16_hi(v[hh].x), bf16_lo(v[hh].y), bf16_hi(v[hh].y),
                          bf16_lo(v[hh].z), bf16_hi(v[hh].z), bf16_lo(v[hh].w), bf16_hi(v[hh].w)};
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
            amax = quad_max(amax);  // all lanes take part (a quad is valid or not as a whole)
            if (tok[hh] < 0) continue;
            const uint32_t b = ue8m0_e4m3(amax);
            uint2 q;
            q.x = pack_fp8x4_scaled(f[0], f[1], f[2], f[3], b);
            q.y = pack_fp8x4_scaled(f[4], f[5], f[6], f[7], b);
            const int64_t t = t0 + tok[hh];
            const int c0 = col[hh];
            if (tok_s && (threadIdx.x & 3) == 0) {
                const int gi = c0 / 32;  // group gi is byte (0, 2, 1, 3)[gi % 4] of word gi / 4
                tok_s[t * (H / 32) + (gi & ~3) + (((gi & 1) << 1) | ((gi >> 1) & 1))] = (uint8_t)b;
            }
            for (int k = 0; k < K; ++k) {
                const int32_t r = rows[tok[hh] * K + k];
                if (r < 0) continue;
                *reinterpret_cast<uint2*>(pool + (int64_t)r * H + c0) = q;
                if (pool_s && (threadIdx.x & 3) == 0) pool_s[(int64_t)r * (H / 32) + c0 / 32] = (uint8_t)b;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_dispatch_fp8(const uint16_t* __restrict__ x, int64_t T,
                                                     int H, int K, int tpb,
                                                     const int32_t* __restrict__ slot_to_pool,
                                                     uint8_t* __restrict__ pool,
                                                     uint8_t* __restrict__ pool_s,
                                                     uint8_t* __restrict__ tok_s) {
    dispatch_fp8_block(x, T, H, K, tpb, slot_to_pool, pool, pool_s, tok_s, blockIdx.x);
}

// The fused layer's first launch: blocks [0, ncount) compute the a1
// histograms (per segment, or with blk_hist set one per block of
// kRouteWaves segments, for k_route), the others quantise the token rows
// token-major (the two are independent, so the histogram hides behind the
// row stream).
__global__ __launch_bounds__(256) void k_quantise_count(const uint16_t* __restrict__ x, int64_t T,
                                                       int H, int tpb, uint8_t* __restrict__ x_q,
                                                       uint8_t* __restrict__ tok_s,
                                                       const int64_t* __restrict__ topk_idx,
                                                       int64_t TK, int E, int ncount,
                                                       int32_t* __restrict__ seg_hist,
                                                       int32_t* __restrict__ seg_err,
                                                       int32_t* __restrict__ blk_hist,
                                                       int32_t* __restrict__ blk_err) {
    extern __shared__ int32_t lds_hist[];  // [kRouteWaves][E]
    if ((int)blockIdx.x < ncount)
        route_count_block(topk_idx, TK, E, seg_hist, seg_err, blockIdx.x, lds_hist, blk_hist, blk_err);
    else
        dispatch_fp8_block(x, T, H, 1, tpb, nullptr, x_q, nullptr, tok_s, blockIdx.x - ncount);
}

// a1-a3 for a batch of at most kRouteWaves * kSegSlots slots, over nb =
// ceil(T*K / 256) blocks of which no block waits for another: block b ranks
// slots [256 b, 256 b + 256) (wave w: 64 of them) and counts every slot of
// the batch itself (at most 1024 indices) for the expert totals, hence the
// offsets, and the expert's rows before its range.  Block 0 also writes the
// tables.  LDS: 7 E counters and kRouteWaves + 1 words.
__device__ __forceinline__ void route_small_block(
    int b, const int64_t* __restrict__ topk_idx, const float* __restrict__ topk_w, int64_t TK, int E,
    int nbits, int K, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    MTile* __restrict__ mtiles, int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag,
    int32_t* __restrict__ pool_src, int32_t* __restrict__ slot_to_pool, float* __restrict__ pool_w,
    int32_t* __restrict__ pool_tok, MTile* __restrict__ mtiles64, int32_t* __restrict__ num_mtiles64,
    int dec_rows, int32_t* lds) {
    int32_t* s_tot = lds;                      // [E] expert totals
    int32_t* s_pre = s_tot + E;                // [E] the expert's slots before this block's range
    int32_t* s_run = s_pre + E;                // [kRouteWaves][E] per-wave counts, then running bases
    int32_t* s_off = s_run + kRouteWaves * E;  // [E] offsets
    int32_t* s_w = s_off + E;                  // [kRouteWaves] scan scratch
    const int tid = threadIdx.x, wv = tid / kWave, lane = tid % kWave;
    const int64_t lo = (int64_t)b * kRouteThreads;
    for (int e = tid; e < 6 * E; e += kRouteThreads) lds[e] = 0;
    // this wave's slot (index and weight)
    const int64_t f = lo + tid;
    int my_e = -1;
    float my_w = 0.f;
    if (f < TK) {
        const int64_t v = topk_idx[f];
        if (v >= 0 && v < E) {
            my_e = (int)v;
            my_w = topk_w[f];
        }
    }
    __syncthreads();
    // every slot of the batch counted
    int bad = 0;
    for (int64_t g = tid; g < TK; g += kRouteThreads) {
        const int64_t v = topk_idx[g];
        if (v >= E) {
            bad = 1;
        } else if (v >= 0) {
            atomicAdd(&s_tot[v], 1);
            if (g < lo)
                atomicAdd(&s_pre[v], 1);
            else if (g < lo + kRouteThreads)
                atomicAdd(&s_run[((g - lo) / kWave) * E + v], 1);
        }
    }
    __syncthreads();
    // offsets, and the running base of each wave: the expert's offset, its
    // slots before this block, then the earlier waves of this block
    const int ept = (E + kRouteThreads - 1) / kRouteThreads;
    int my_tot = 0;
    for (int j = 0; j < ept; ++j) {
        const int e = ept * tid + j;
        if (e < E) my_tot += s_tot[e];
    }
    int R = 0;
    int off = block_exclusive_scan(my_tot, &R, s_w);
    for (int j = 0; j < ept; ++j) {
        const int e = ept * tid + j;
        if (e >= E) continue;
        s_off[e] = off;
        int run = off + s_pre[e];
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            const int c = s_run[w * E + e];
            s_run[w * E + e] = run;
            run += c;
        }
        off += s_tot[e];
    }
    __syncthreads();
    // the stable rank of the wave's slot: lanes holding the same expert find
    // each other with one ballot per index bit, the lower lanes first
    if (f - lane < TK) {  // wave-uniform: the wave's first slot exists
        unsigned long long peers = __ballot(my_e >= 0);
        for (int bt = 0; bt < nbits; ++bt) {
            const int bit = (my_e >> bt) & 1;
            const unsigned long long set = __ballot(bit);
            peers &= bit ? set : ~set;
        }
        if (my_e >= 0) {
            const int r = s_run[wv * E + my_e] + __popcll(peers & ((1ull << lane) - 1ull));
            pool_src[r] = (int32_t)f;
            slot_to_pool[f] = r;
            pool_w[r] = my_w;
            pool_tok[r] = (int32_t)(f / K);
        } else if (f < TK) {
            slot_to_pool[f] = -1;
        }
    }
    if (b == 0) {
        const int err = __syncthreads_or(bad);
        route_write_tables(E, R, err, s_tot, s_off, s_w, counts, offsets, mtiles, num_mtiles, err_flag,
                           mtiles64, num_mtiles64, dec_rows);
    }
}

// The fused layer's first launch for batches of at most kRouteWaves *
// kSegSlots slots: blocks [0, nroute) route (route_small_block), the others
// quantise the token rows token-major.  The pool rows' A-scale words need
// every token's words, so they are not gathered here.
__global__ __launch_bounds__(256) void k_quantise_route(
    const uint16_t* __restrict__ x, int64_t T, int H, int tpb, uint8_t* __restrict__ x_q,
    uint8_t* __restrict__ tok_s, const int64_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, int64_t TK, int E, int nbits, int K, int nroute,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, MTile* __restrict__ mtiles,
    int32_t* __restrict__ num_mtiles, int32_t* __restrict__ err_flag,
    int32_t* __restrict__ pool_src, int32_t* __restrict__ slot_to_pool, float* __restrict__ pool_w,
    int32_t* __restrict__ pool_tok, MTile* __restrict__ mtiles64, int32_t* __restrict__ num_mtiles64,
    int dec_rows) {
    extern __shared__ int32_t lds[];
    if ((int)blockIdx.x < nroute)
        route_small_block(blockIdx.x, topk_idx, topk_w, TK, E, nbits, K, counts, offsets, mtiles, num_mtiles,
                          err_flag, pool_src, slot_to_pool, pool_w, pool_tok, mtiles64, num_mtiles64, dec_rows,
                          lds);
    else
        dispatch_fp8_block(x, T, H, 1, tpb, nullptr, x_q, nullptr, tok_s, blockIdx.x - nroute);
}

// A-scale words of the pool rows in packed k-major order (the layout the L1
// GEMM loads per K step: word (w, r) at 4 * (w * cap + r)), gathered from the
// token-major words the dispatch wrote (already in the byte order 0, 2, 1,
// 3): word (w, r) = word w of token pool_tok[r].  Thread per pool row; the
// token's words are read as 16-byte pieces, and for each w consecutive threads
// write consecutive words.  Rows from R on are left as they are.
__global__ __launch_bounds__(256) void k_pool_scales(const uint32_t* __restrict__ tok_s, int W,
                                                    const int32_t* __restrict__ pool_tok,
                                                    const int32_t* __restrict__ offsets, int E,
                                                    int64_t cap, uint32_t* __restrict__ pool_s) {
    const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (r >= offsets[E]) return;
    const int64_t t = pool_tok[r];
    if ((W & 3) == 0) {
        const uint4* src = reinterpret_cast<const uint4*>(tok_s + t * W);
        for (int w4 = 0; w4 < W / 4; ++w4) {
            const uint4 v = src[w4];
            pool_s[(int64_t)(4 * w4 + 0) * cap + r] = v.x;
            pool_s[(int64_t)(4 * w4 + 1) * cap + r] = v.y;
            pool_s[(int64_t)(4 * w4 + 2) * cap + r] = v.z;
            pool_s[(int64_t)(4 * w4 + 3) * cap + r] = v.w;
        }
    } else {
        for (int w = 0; w < W; ++w) pool_s[(int64_t)w * cap + r] = tok_s[t * W + w];
    }
}

// Weight scales [E][N][W words] (row-major, W = Kdim/128 words of 4 UE8M0
// bytes per row) -> packed k-major [E][W][N], bytes in the order 0, 2, 1, 3.
// Block (n-tile of 64 rows, expert, word tile of 64): 16-byte row reads into
// an LDS tile, 16-byte column writes (4 rows of one word) out of it.
__global__ __launch_bounds__(256) void k_scales_kmajor(const uint32_t* __restrict__ S,
                                                      uint32_t* __restrict__ St, int N, int W) {
    __shared__ uint32_t tile[64][64 + 4];
    const int n0 = blockIdx.x * 64, e = blockIdx.y, w0 = blockIdx.z * 64;
    const int nw = min(64, W - w0);
    const uint32_t* src = S + ((int64_t)e * N + n0) * W + w0;
    if ((W & 3) == 0) {  // rows are 16-byte aligned
        for (int i = threadIdx.x; i < 64 * 16; i += 256) {
            const int r = i >> 4, w4 = i & 15;
            if (4 * w4 < nw) {
                const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)r * W + 4 * w4);
                tile[4 * w4 + 0][r] = v.x;
                tile[4 * w4 + 1][r] = v.y;
                tile[4 * w4 + 2][r] = v.z;
                tile[4 * w4 + 3][r] = v.w;
            }
        }
    } else {
        for (int i = threadIdx.x; i < 64 * 64; i += 256) {
            const int r = i >> 6, w = i & 63;
            if (w < nw) tile[w][r] = src[(int64_t)r * W + w];
        }
    }
    __syncthreads();
    uint32_t* dst = St + ((int64_t)e * W + w0) * N + n0;
    for (int i = threadIdx.x; i < 64 * 16; i += 256) {
        const int w = i >> 4, r4 = i & 15;
        if (w < nw) {
            uint4 v;
            v.x = swap_bytes12(tile[w][4 * r4 + 0]);
            v.y = swap_bytes12(tile[w][4 * r4 + 1]);
            v.z = swap_bytes12(tile[w][4 * r4 + 2]);
            v.w = swap_bytes12(tile[w][4 * r4 + 3]);
            *reinterpret_cast<uint4*>(dst + (int64_t)w * N + 4 * r4) = v;
        }
    }
}

// a4 with a bf16 payload: plain row copies (for callers that run their own
// expert GEMM on bf16 rows).
__global__ __launch_bounds__(256) void k_dispatch_bf16(const uint16_t* __restrict__ x, int H,
                                                      int K, const int32_t* __restrict__ slot_to_pool,
                                                      uint16_t* __restrict__ pool) {
    __shared__ int32_t rows[64];
    const int64_t t = blockIdx.x;
    if (threadIdx.x < K) rows[threadIdx.x] = slot_to_pool[t * K + threadIdx.x];
    __syncthreads();
    const uint16_t* xr = x + t * H;
    for (int c0 = threadIdx.x * 8; c0 < H; c0 += 256 * 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(xr + c0);
        for (int k = 0; k < K; ++k) {
            const int32_t r = rows[k];
            if (r >= 0) *reinterpret_cast<uint4*>(pool + (int64_t)r * H + c0) = v;
        }
    }
}

// a9: combine.  A group of tpb consecutive tokens (tpb * H <= 8192 when
// tpb > 1, so that small rows still fill a block) goes to nparts blocks, each
// taking one piece of the group's flat [tpb][H] columns (nparts > 1 only for
// small batches, whose groups alone would not cover the GPU); each lane owns
// 8 columns of up to four 2048-column chunks of its block's piece.
// The K pool rows behind every chunk are loaded first (4K independent loads
// in flight per lane, the rate of a plain HBM read stream), then summed in
// ascending k in fp32 starting from +0, then rounded to bf16.  Multiplies and
// adds stay separately rounded.
// 2048-column chunks per lane per pass (each with its K rows' loads in flight)
constexpr int kCH = 4;
#pragma clang fp contract(off)
__global__ __launch_bounds__(256) void k_combine(const uint16_t* __restrict__ o,
                                                const int32_t* __restrict__ slot_to_pool,
                                                const float* __restrict__ topk_w, int64_t T,
                                                int H, int K, int tpb, int nparts,
                                                uint16_t* __restrict__ y) {
    __shared__ int32_t rows[kMaxBlockTokens * 64];
    __shared__ float wts[kMaxBlockTokens * 64];
    const int part = (int)(blockIdx.x % (unsigned)nparts);
    const int64_t t0 = (int64_t)(blockIdx.x / (unsigned)nparts) * tpb;
    for (int i = threadIdx.x; i < tpb * K; i += 256) {
        const int64_t t = t0 + i / K;
        const bool in = t < T;
        rows[i] = in ? slot_to_pool[t0 * K + i] : -1;
        wts[i] = (in && topk_w) ? topk_w[t0 * K + i] : 1.0f;
    }
    __syncthreads();
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    // the block's share of the flat columns of its tokens: part `part` of
    // nparts pieces of whole 8-column runs
    const int span = tpb * H;
    const int piece = ((span + nparts - 1) / nparts + 7) & ~7;
    const int lo = part * piece, hi = min(span, lo + piece);
    for (int c00 = lo + threadIdx.x * 8; c00 < hi; c00 += kCH * 256 * 8) {
        int tok[kCH], col[kCH];
#pragma unroll
        for (int hh = 0; hh < kCH; ++hh) {
            const int p = c00 + hh * 256 * 8;
            const int j = p < hi ? p / H : -1;  // H % 8 == 0: a lane's 8 columns share a token
            tok[hh] = j;
            col[hh] = j >= 0 ? p - j * H : 0;
        }
        float acc[kCH][8];
#pragma unroll
        for (int hh = 0; hh < kCH; ++hh)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[hh][j] = 0.0f;
        for (int k0 = 0; k0 < K; k0 += 8) {
            u32x4 v[kCH][8];
#pragma unroll
            for (int hh = 0; hh < kCH; ++hh) {
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int k = k0 + u;
                    const int32_t r = (k < K && tok[hh] >= 0) ? rows[tok[hh] * K + k] : -1;
                    // streamed: each L2 output byte is read exactly once
                    const u32x4 z = {0, 0, 0, 0};
                    v[hh][u] = r >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                            o + (int64_t)r * H + col[hh]))
                                      : z;
                }
            }
#pragma unroll
            for (int hh = 0; hh < kCH; ++hh) {
                if (tok[hh] < 0) continue;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int k = k0 + u;
                    if (k >= K || rows[tok[hh] * K + k] < 0) continue;
                    const uint32_t w4[4] = {v[hh][u].x, v[hh][u].y, v[hh][u].z, v[hh][u].w};
                    if (topk_w) {
                        const float wk = wts[tok[hh] * K + k];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[hh][2 * j] = acc[hh][2 * j] + bf16_lo(w4[j]) * wk;
                            acc[hh][2 * j + 1] = acc[hh][2 * j + 1] + bf16_hi(w4[j]) * wk;
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            acc[hh][2 * j] = acc[hh][2 * j] + bf16_lo(w4[j]);
                            acc[hh][2 * j + 1] = acc[hh][2 * j + 1] + bf16_hi(w4[j]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int hh = 0; hh < kCH; ++hh) {
            if (tok[hh] < 0 || t0 + tok[hh] >= T) continue;
            const u32x4 out = {pack_bf16x2(acc[hh][0], acc[hh][1]), pack_bf16x2(acc[hh][2], acc[hh][3]),
                               pack_bf16x2(acc[hh][4], acc[hh][5]), pack_bf16x2(acc[hh][6], acc[hh][7])};
            __builtin_nontemporal_store(
                out, reinterpret_cast<u32x4*>(y + (t0 + tok[hh]) * H + col[hh]));  // streamed out
        }
    }
}

}  // namespace moe
