// Online block routing for Sol-Attn on gfx950: block-mean pooling of Q and K,
// pooled scores in a fixed float32 order, and per-query-block selection under
// threshold tau with the diagonal forced, written as compact ascending lists.
//
// Routing from compressed queries and keys under tau with a "diagonal
// threshold" is named on the clawpit.io article (paragraph on the Sol-Attn
// settings) and the nvlabs Sol-Engine H3 page (policy paragraph); the pages
// give no formula.  The rule implemented (gap to the row maximum, diagonal
// always kept) and its exact float32 order are stated in include/sol.h.
//
// Two kernels:
//   pool_kernel          HBM-bound scan of K (and of Q when routing from
//                        means is not fused, see below; each element read
//                        once); one lane owns 8 channels of one head and adds
//                        the block's rows in ascending order.
//   score_select_kernel  one lane owns one candidate key block (or a few) and
//                        the workgroup's 12 or 16 query blocks, whose pooled
//                        rows sit in LDS; the channels go in 8-wide chunks;
//                        each score is an FMA chain over d ascending.  In
//                        sol_route the workgroup pools its query blocks from
//                        Q itself (the same order as pool_kernel), so the scan
//                        of Q overlaps other workgroups' scoring.
#include "sol_internal.h"

namespace sol {

namespace {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16 bytes of a row that is read exactly once: a non-temporal load, so the
// streamed Q and K do not displace cached lines (7% faster pooling)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ void add8(float (&acc)[8], const uint4& w) {
    acc[0] += bf_lo(w.x); acc[1] += bf_hi(w.x);
    acc[2] += bf_lo(w.y); acc[3] += bf_hi(w.y);
    acc[4] += bf_lo(w.z); acc[5] += bf_hi(w.z);
    acc[6] += bf_lo(w.w); acc[7] += bf_hi(w.w);
}

// grid: x = token block, y = lane groups of 256 over H * D / 8, z = batch * 2 + (0: Q, 1: K),
// or z = batch with k_only (the Q means are then pooled by the scoring kernel)
// qbar: [B, H, NB, D] float32; kbar: [B, H, D / 8, NB, 8] float32 (8-channel
// chunks, so a lane owning one key block reads its chunk contiguously).
__global__ __launch_bounds__(256) void pool_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, Geom g,
    float* __restrict__ qbar, float* __restrict__ kbar, int k_only)
{
    const int blk = blockIdx.x;
    const int b = k_only ? (int)blockIdx.z : (int)(blockIdx.z >> 1);
    const int is_k = k_only ? 1 : (int)(blockIdx.z & 1);
    const int chunks = g.D >> 3;
    const int lane_id = blockIdx.y * 256 + threadIdx.x;
    if (lane_id >= g.H * chunks) return;
    const Seq sq = seq_of(g, b);
    if (blk >= sq.NB) return;                  // past this sample's last block
    const int h = lane_id / chunks, c = lane_id - h * chunks;
    int r0 = blk * kBlock;
    const int r1 = min(r0 + kBlock, sq.N);
    if (is_k) {
        if (blk < sq.j0) return;
        r0 = max(r0, g.S);
    }
    const uint16_t* src = (is_k ? k : q) + sq.base + (int64_t)h * g.sh + c * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int t = r0;
    // rows strictly in ascending order; loads are issued 16 ahead
    for (; t + 16 <= r1; t += 16) {
        uint4 w[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
            w[u] = load_stream16(src + (int64_t)(t + u) * g.sn);
#pragma unroll
        for (int u = 0; u < 16; ++u) add8(acc, w[u]);
    }
    for (; t < r1; ++t) add8(acc, load_stream16(src + (int64_t)t * g.sn));
    const float rows = (float)(r1 - r0);
    const int64_t bh = (int64_t)b * g.H + h;
    if (!is_k) {
        float4* dst = (float4*)(qbar + (bh * g.NB + blk) * g.D + c * 8);
        dst[0] = make_float4(acc[0] / rows, acc[1] / rows, acc[2] / rows, acc[3] / rows);
        dst[1] = make_float4(acc[4] / rows, acc[5] / rows, acc[6] / rows, acc[7] / rows);
    } else {
        float4* dst = (float4*)(kbar + ((bh * chunks + c) * g.NB + blk) * 8);
        dst[0] = make_float4(acc[0] / rows, acc[1] / rows, acc[2] / rows, acc[3] / rows);
        dst[1] = make_float4(acc[4] / rows, acc[5] / rows, acc[6] / rows, acc[7] / rows);
    }
}

// reductions over the 64 lanes of a wave, result in every lane: DPP within
// rows of 16 lanes, then a swizzle across 16 and a permlane swap across 32
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float swz16(float v) {       // lane ^ 16 within each 32
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ uint32_t swz16(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp<0xB1>(v));      // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));      // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v));     // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v));     // row_mirror
    v = fmaxf(v, swz16(v));
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    v += swz16(v);
    const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return sw[0] + sw[1];
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

constexpr int kMaxWaves = 16;

// query blocks per scoring workgroup when it pools them itself
#ifndef SOL_POOLQ_TI
#define SOL_POOLQ_TI 12
#endif

// grid: x = query-block tiles of TI (XCD-remapped together with y), y = B * H
// block: 64 * W threads; lane slot s = jj * 64 W + tid owns candidate j = j0 + s.
// POOLQ: the workgroup pools its own TI query blocks from q (same order and
// arithmetic as pool_kernel) instead of reading q-bar, so the HBM-bound scan
// of Q runs in workgroups that overlap the VALU-bound scoring of others.
template <int D, int JPL, int TI, bool POOLQ>
__global__ __launch_bounds__(64 * kMaxWaves) void score_select_kernel(
    const float* __restrict__ qbar, const uint16_t* __restrict__ q, const float* __restrict__ kbar,
    Geom g, float scale, float tau, int tiles_per_bh, int16_t* __restrict__ idx,
    int32_t* __restrict__ cnt, unsigned long long* __restrict__ wg_part)
{
    const int work = xcd_remap(blockIdx.x, gridDim.x, tiles_per_bh * g.B * g.H);
    if (work < 0) return;
    const int bh = work / tiles_per_bh;
    const int i0 = (work - bh * tiles_per_bh) * TI;
    const int W = blockDim.x >> 6;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int slots = 64 * W;
    const Seq sq = seq_of(g, bh / g.H);
    // query blocks of this tile inside the sample; the tile's rows past the
    // sample's last block (packed batches) get empty lists
    const int ni = min(TI, sq.NB - i0);
    if (tid < min(TI, g.NB - i0) && tid >= ni) cnt[(int64_t)bh * g.NB + i0 + tid] = 0;
    if (ni <= 0) {                     // nothing routed here: this workgroup's totals are zero
        if (tid == 0) {
            wg_part[2 * work] = 0;
            wg_part[2 * work + 1] = 0;
        }
        return;
    }

    __shared__ float red[TI][kMaxWaves];
    __shared__ int woffset[TI][JPL * kMaxWaves];

    const float* qb = qbar + (int64_t)bh * g.NB * D;
    const float* kb = kbar + (int64_t)bh * (D / 8) * g.NB * 8;

    // scores: each lane owns JPL candidates and the TI query blocks of the
    // workgroup.  The TI pooled query rows are staged in LDS once and read
    // back as broadcasts; the channels go in 8-wide chunks, so a lane loads
    // 32 bytes of k-bar per chunk and each q-bar value feeds JPL FMAs.  Every
    // score is still one FMA chain over d ascending.
    __shared__ __attribute__((aligned(16))) float qs[TI][D];
    // the workgroup's totals, written to its own slot of wg_part and summed by
    // totals_kernel afterwards (one global atomic per workgroup on the same
    // two counters was 6% of routing time)
    __shared__ unsigned long long wg_tot[2];
    if (tid == 0) {
        wg_tot[0] = 0;
        wg_tot[1] = 0;
    }
    if constexpr (POOLQ) {
        // one (query block, 8-channel chunk) per lane and pass: the block's
        // valid rows added in ascending order, loads issued 16 ahead, one
        // divide -- the q-bar of pool_kernel, bit for bit
        constexpr int CH = D / 8;
        const uint16_t* qsrc = q + sq.base + (int64_t)(bh % g.H) * g.sh;
        for (int e = tid; e < TI * CH; e += blockDim.x) {
            const int ii = e / CH, c = e - ii * CH;
            float a8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float rows = 1.f;
            if (ii < ni) {
                const int r0 = (i0 + ii) * kBlock;
                const int r1 = min(r0 + kBlock, sq.N);
                const uint16_t* src = qsrc + c * 8;
                int t = r0;
                for (; t + 16 <= r1; t += 16) {
                    uint4 w[16];
#pragma unroll
                    for (int u = 0; u < 16; ++u)
                        w[u] = load_stream16(src + (int64_t)(t + u) * g.sn);
#pragma unroll
                    for (int u = 0; u < 16; ++u) add8(a8, w[u]);
                }
                for (; t < r1; ++t) add8(a8, load_stream16(src + (int64_t)t * g.sn));
                rows = (float)(r1 - r0);
            }
#pragma unroll
            for (int x = 0; x < 8; ++x) qs[ii][8 * c + x] = a8[x] / rows;
        }
    } else {
        for (int e = tid; e < TI * D; e += blockDim.x) {
            const int ii = e / D;
            qs[ii][e - ii * D] = ii < ni ? qb[(int64_t)(i0 + ii) * D + (e - ii * D)] : 0.f;
        }
    }
    __syncthreads();
    int jrow[JPL];
    bool jvalid[JPL];
    float acc[JPL][TI];
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj) {
        const int s = jj * slots + tid;
        jvalid[jj] = s < sq.ncand;
        // slots past the candidates read row 0 (always inside the workspace,
        // even when the sample has no candidate) and score -inf below
        jrow[jj] = jvalid[jj] ? sq.j0 + s : 0;
#pragma unroll
        for (int ii = 0; ii < TI; ++ii) acc[jj][ii] = 0.f;
    }
    for (int c = 0; c < D / 8; ++c) {
        float kv[JPL][8];
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) {
            const float4* p = (const float4*)(kb + ((int64_t)c * g.NB + jrow[jj]) * 8);
            const float4 a = p[0], b = p[1];
            kv[jj][0] = a.x; kv[jj][1] = a.y; kv[jj][2] = a.z; kv[jj][3] = a.w;
            kv[jj][4] = b.x; kv[jj][5] = b.y; kv[jj][6] = b.z; kv[jj][7] = b.w;
        }
#pragma unroll
        for (int ii = 0; ii < TI; ++ii) {
            const float4 qa = *(const float4*)&qs[ii][8 * c];
            const float4 qc = *(const float4*)&qs[ii][8 * c + 4];
            const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qc.x, qc.y, qc.z, qc.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int jj = 0; jj < JPL; ++jj)
                    acc[jj][ii] = __builtin_fmaf(qv[e], kv[jj][e], acc[jj][ii]);
        }
    }
    float sc[JPL][TI];
#pragma unroll
    for (int jj = 0; jj < JPL; ++jj)
#pragma unroll
        for (int ii = 0; ii < TI; ++ii) sc[jj][ii] = jvalid[jj] ? acc[jj][ii] * scale : -INFINITY;

    // row maxima over all candidates of the workgroup
#pragma unroll
    for (int ii = 0; ii < TI; ++ii) {
        float m = sc[0][ii];
#pragma unroll
        for (int jj = 1; jj < JPL; ++jj) m = fmaxf(m, sc[jj][ii]);
        m = wave_max(m);
        if (lane == 0) red[ii][wave] = m;
    }
    __syncthreads();
    float thr[TI];
#pragma unroll
    for (int ii = 0; ii < TI; ++ii) {
        float m = red[ii][0];
        for (int w = 1; w < W; ++w) m = fmaxf(m, red[ii][w]);
        thr[ii] = m - tau;
    }

    // selection.  Pass 1: each wave's ballot per (query block, candidate
    // slot) goes to LDS, and each lane sums the attended (row, key) pairs of
    // its selected candidates.
    __shared__ unsigned long long balls[TI][JPL * kMaxWaves];
    // each lane also keeps its own selections as bits ii * JPL + jj, so the
    // compaction below rebuilds the ballots instead of reading them back
    static_assert(TI * JPL <= 64, "one selection bit per (query block, slot)");
    uint64_t selbits = 0;
    uint32_t keys_local = 0;
#pragma unroll
    for (int ii = 0; ii < TI; ++ii) {
        const int i = i0 + ii;
        const uint32_t rows = (uint32_t)max(min(kBlock, sq.N - kBlock * i), 0);
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) {
            const int sl = jj * slots + tid;
            const int j = sq.j0 + sl;
            const bool sel = (ii < ni) && jvalid[jj] && (sc[jj][ii] >= thr[ii] || j == i);
            const uint64_t bal = __ballot(sel);
            if (lane == 0) balls[ii][jj * W + wave] = bal;
            selbits |= (uint64_t)(sel ? 1 : 0) << (ii * JPL + jj);
            const uint32_t keys = (uint32_t)(min(kBlock * j + kBlock, sq.N) - max(kBlock * j, g.S));
            keys_local += sel ? rows * keys : 0u;
        }
    }
    __syncthreads();
    // counts and list offsets: one thread per query block
    if (tid < ni) {
        int run = 0;
        for (int e = 0; e < JPL * W; ++e) {
            woffset[tid][e] = run;
            run += __popcll(balls[tid][e]);
        }
        cnt[(int64_t)bh * g.NB + i0 + tid] = run;
        const int rows = min(kBlock, sq.N - kBlock * (i0 + tid));
        atomicAdd(&wg_tot[0], (unsigned long long)run);
        atomicAdd(&wg_tot[1], (unsigned long long)rows * sq.Ssink);
    }
    __syncthreads();
    // pass 2: compaction into ascending lists (slot order = block order).
    // Lane e fetches this wave's list offset of (query block e / JPL, slot
    // e % JPL) in one LDS read; the loop takes it back with readlane.
    int my_off = 0;
    if (lane < TI * JPL && lane / JPL < ni) my_off = woffset[lane / JPL][(lane % JPL) * W + wave];
#pragma unroll
    for (int ii = 0; ii < TI; ++ii) {
        if (ii >= ni) break;
        int16_t* row = idx + ((int64_t)bh * g.NB + i0 + ii) * g.NB;
#pragma unroll
        for (int jj = 0; jj < JPL; ++jj) {
            const bool sel = (selbits >> (ii * JPL + jj)) & 1;
            const uint64_t bal = __ballot(sel);
            const int off = __builtin_amdgcn_readlane(my_off, ii * JPL + jj);
            if (sel) row[off + lanes_below(bal)] = (int16_t)(sq.j0 + jj * slots + tid);
        }
    }
    const uint32_t wsum = wave_sum(keys_local);
    if (lane == 0 && wsum != 0) atomicAdd(&wg_tot[1], (unsigned long long)wsum);
    __syncthreads();
    if (tid == 0) {
        wg_part[2 * work] = wg_tot[0];
        wg_part[2 * work + 1] = wg_tot[1];
    }
}

// S >= N: no candidates, every list is empty, only sink pairs are attended;
// the schedule is sequence order.  Workgroup 0 also sums the sink pairs of
// every sample (rows x sink keys, per head).
__global__ __launch_bounds__(256) void empty_route_kernel(int32_t* __restrict__ cnt, Geom g,
                                                          int64_t* __restrict__ totals,
                                                          int32_t* __restrict__ order)
{
    const int n = g.B * g.H * g.NB;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        cnt[i] = 0;
        if (order != nullptr) order[i] = i % g.NB;
    }
    if (blockIdx.x == 0) {
        __shared__ unsigned long long part[256];
        unsigned long long acc = 0;
        for (int b = threadIdx.x; b < g.B; b += 256) {
            const Seq sq = seq_of(g, b);
            acc += (unsigned long long)g.H * sq.N * sq.Ssink;
        }
        part[threadIdx.x] = acc;
        __syncthreads();
        for (int off = 128; off > 0; off >>= 1) {
            if (threadIdx.x < off) part[threadIdx.x] += part[threadIdx.x + off];
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            totals[0] = 0;
            totals[1] = (int64_t)part[0];
        }
    }
}

// totals = the sum of the scoring workgroups' partial totals (one workgroup)
__global__ __launch_bounds__(256) void totals_kernel(const unsigned long long* __restrict__ wg_part,
                                                     int n, int64_t* __restrict__ totals)
{
    __shared__ unsigned long long part[2][256];
    unsigned long long a = 0, b = 0;
    for (int i = threadIdx.x; i < n; i += 256) {
        a += wg_part[2 * i];
        b += wg_part[2 * i + 1];
    }
    part[0][threadIdx.x] = a;
    part[1][threadIdx.x] = b;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) {
            part[0][threadIdx.x] += part[0][threadIdx.x + off];
            part[1][threadIdx.x] += part[1][threadIdx.x + off];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        totals[0] = (int64_t)part[0][0];
        totals[1] = (int64_t)part[1][0];
    }
}

// Attention schedule: the query blocks of each (batch, head) sorted by list
// length, longest first (a counting sort over the lengths 0..ncand).  Running
// the long walks first balances the tail of the attention launch, and query
// blocks running side by side then have lists of similar length, so their
// ascending walks sweep the key blocks at similar rates and share them in L2.
// Blocks of equal length keep no particular order; each query block's output
// does not depend on the order, only the timing does.
// A packed sample sorts its own blocks; the row's entries past them hold
// their own index.
// grid: B * H; block: 256; dynamic LDS: ncand + 1 ints (ncand of the call).
__global__ __launch_bounds__(256) void order_kernel(const int32_t* __restrict__ cnt, Geom g,
                                                    int32_t* __restrict__ order)
{
    extern __shared__ int hist[];          // per list length: count, then next slot
    __shared__ int part[256];
    const int tid = threadIdx.x;
    const Seq sq = seq_of(g, blockIdx.x / g.H);
    const int ncand = sq.ncand, NB = sq.NB;
    const int nbins = ncand + 1;
    const int64_t row = (int64_t)blockIdx.x * g.NB;
    for (int i = NB + tid; i < g.NB; i += 256) order[row + i] = i;
    for (int b = tid; b < nbins; b += 256) hist[b] = 0;
    __syncthreads();
    for (int i = tid; i < NB; i += 256) atomicAdd(&hist[min(max(cnt[row + i], 0), ncand)], 1);
    __syncthreads();
    // descending exclusive scan: thread t owns lengths ncand - k for k in its range
    const int per = (nbins + 255) / 256;
    const int k0 = min(tid * per, nbins), k1 = min(k0 + per, nbins);
    int local = 0;
    for (int kk = k0; kk < k1; ++kk) local += hist[ncand - kk];
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {      // inclusive Hillis-Steele scan
        const int add = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    int run = part[tid] - local;
    for (int kk = k0; kk < k1; ++kk) {
        const int b = ncand - kk;
        const int n = hist[b];
        hist[b] = run;
        run += n;
    }
    __syncthreads();
    for (int i = tid; i < NB; i += 256) {
        const int pos = atomicAdd(&hist[min(max(cnt[row + i], 0), ncand)], 1);
        order[row + pos] = i;
    }
}

template <int D>
hipError_t launch_select(const Geom& g, const float* qbar, const uint16_t* q, const float* kbar,
                         float scale, float tau, int16_t* idx, int32_t* cnt, int64_t* totals,
                         unsigned long long* wg_part, hipStream_t stream)
{
    // candidates per lane (1, 2, 4 or 5): each q-bar value read from LDS
    // feeds that many FMAs.  The candidates fill whole waves of 64 lanes, so
    // the count is chosen to leave the fewest lanes on padding (the score
    // pass is bound by its VALU FMAs, padded ones included): at 584
    // candidates 5 per lane fill 2 waves x 320 slots (91%), where 4 per lane
    // would fill 3 waves x 256 (76%).  Ties go to the larger count.  16 waves
    // x 64 lanes x 4 cover the 4096-candidate limit.  Query blocks per
    // workgroup: 12 with 4 or 5 candidates per lane (each k-bar chunk a lane
    // loads feeds 12 x 8 x JPL FMAs), 16 otherwise.
    int jpl = 1;
    if (g.ncand > 64) {
        long best = -1;
        for (const int j : {2, 4, 5}) {
            const long w = (g.ncand + 64 * j - 1) / (64 * j);
            const long slots = w * 64 * j;
            if (w <= kMaxWaves && (best < 0 || slots <= best)) {
                best = slots;
                jpl = j;
            }
        }
    }
    const int W = (g.ncand + 64 * jpl - 1) / (64 * jpl);
#define SOL_SELECT_CASE(J, T, P)                                                            \
    do {                                                                                    \
        const int tiles = (g.NB + (T) - 1) / (T);                                           \
        const int total = tiles * g.B * g.H;                                                \
        const int grid = round_up(total, kXcds);                                            \
        hipLaunchKernelGGL((score_select_kernel<D, J, T, P>), dim3(grid), dim3(64 * W), 0,  \
                           stream, qbar, q, kbar, g, scale, tau, tiles, idx, cnt, wg_part); \
        works = total;                                                                      \
    } while (0)
    int works = 0;
    if (q != nullptr) {
        // pooling its own query blocks: SOL_POOLQ_TI of them per workgroup
        if (jpl == 1) SOL_SELECT_CASE(1, SOL_POOLQ_TI, true);
        else if (jpl == 2) SOL_SELECT_CASE(2, SOL_POOLQ_TI, true);
        else if (jpl == 4) SOL_SELECT_CASE(4, SOL_POOLQ_TI, true);
        else SOL_SELECT_CASE(5, SOL_POOLQ_TI, true);
    } else {
        if (jpl == 1) SOL_SELECT_CASE(1, 16, false);
        else if (jpl == 2) SOL_SELECT_CASE(2, 16, false);
        else if (jpl == 4) SOL_SELECT_CASE(4, 12, false);
        else SOL_SELECT_CASE(5, 12, false);
    }
#undef SOL_SELECT_CASE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(totals_kernel, dim3(1), dim3(256), 0, stream, wg_part, works, totals);
    return hipGetLastError();
}

// scores and selection from the block means, then the schedule
hipError_t select_and_order(const Geom& g, const float* qbar, const uint16_t* q,
                            const float* kbar, float scale, float tau, int16_t* idx, int32_t* cnt,
                            int64_t* totals, int32_t* order, unsigned long long* wg_part,
                            hipStream_t stream)
{
    hipError_t e = g.D == 128
        ? launch_select<128>(g, qbar, q, kbar, scale, tau, idx, cnt, totals, wg_part, stream)
        : launch_select<64>(g, qbar, q, kbar, scale, tau, idx, cnt, totals, wg_part, stream);
    if (e != hipSuccess || order == nullptr) return e;
    hipLaunchKernelGGL(order_kernel, dim3(g.B * g.H), dim3(256), (size_t)(g.ncand + 1) * sizeof(int),
                       stream, cnt, g, order);
    return hipGetLastError();
}

}  // namespace

// partial totals of the scoring workgroups: two uint64 per workgroup, at most
// ceil(NB / min tile) workgroups per (batch, head)
static size_t part_floats(const Geom& g) {
    constexpr int kMinTile = SOL_POOLQ_TI < 12 ? SOL_POOLQ_TI : 12;
    const size_t works = (size_t)((g.NB + kMinTile - 1) / kMinTile) * g.B * g.H;
    return (4 * works + 63) / 64 * 64;
}

size_t route_ws_floats(const Geom& g) {
    // qbar and kbar, each B * H * NB * D floats rounded to 64 floats, then the
    // scoring workgroups' partial totals
    const size_t one = (size_t)g.B * g.H * g.NB * g.D;
    return 2 * ((one + 63) / 64 * 64) + part_floats(g);
}

hipError_t launch_route(const Geom& g, const void* q, const void* k, float scale, float tau,
                        int16_t* idx, int32_t* cnt, int64_t* totals, int32_t* order, float* ws,
                        hipStream_t stream)
{
    if (g.ncand == 0) {
        const int n = g.B * g.H * g.NB;
        hipLaunchKernelGGL(empty_route_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, cnt, g,
                           totals, order);
        return hipGetLastError();
    }
    const size_t one = ((size_t)g.B * g.H * g.NB * g.D + 63) / 64 * 64;
    float* qbar = ws;
    float* kbar = ws + one;
    const int lanes = g.H * (g.D / 8);
    // the K means here; the scoring workgroups pool their own query blocks
    dim3 grid(g.NB, (lanes + 255) / 256, g.B);
    hipLaunchKernelGGL(pool_kernel, grid, dim3(256), 0, stream, (const uint16_t*)q,
                       (const uint16_t*)k, g, qbar, kbar, 1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return select_and_order(g, qbar, (const uint16_t*)q, kbar, scale, tau, idx, cnt, totals, order,
                            reinterpret_cast<unsigned long long*>(ws + 2 * one), stream);
}

hipError_t launch_route_pooled(const Geom& g, float scale, float tau, int16_t* idx, int32_t* cnt,
                               int64_t* totals, int32_t* order, float* ws, hipStream_t stream)
{
    if (g.ncand == 0) {
        const int n = g.B * g.H * g.NB;
        hipLaunchKernelGGL(empty_route_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, cnt, g,
                           totals, order);
        return hipGetLastError();
    }
    const size_t one = ((size_t)g.B * g.H * g.NB * g.D + 63) / 64 * 64;
    return select_and_order(g, ws, nullptr, ws + one, scale, tau, idx, cnt, totals, order,
                            reinterpret_cast<unsigned long long*>(ws + 2 * one), stream);
}

}  // namespace sol
