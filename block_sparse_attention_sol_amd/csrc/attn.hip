// Sol-Attn block-sparse attention forward on gfx950: exact prefix sink plus the
// routed key blocks of each 64-token query block, one online softmax over
// both (the exact log-sum-exp merge of the sink and routed parts), bf16 MFMA
// with float32 accumulation.
//
// The sink / routed split follows the nvlabs Sol-Engine H3 page (policy
// paragraph: exact 951-token prefix sink, online routing) and the clawpit.io
// article (paragraph on the Sol-Attn settings).  Because the sink keys and the
// routed keys are disjoint, running one online softmax over the sink tiles and
// then the routed tiles gives exactly the log-sum-exp merge of the two parts.
//
// Work decomposition: one wave per (batch, head, query block), 64 query rows.
// Per 64-key tile the wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = K straight from global memory into registers, B = Q^T held in
// registers for the whole walk), so each lane ends up holding 32 scores of
// one query row; the softmax row statistics need a single cross-lane step
// (lane l and l ^ 32 share a row).  Then O^T += V^T P^T: P comes from the score
// registers as the B operand with no data movement, and V^T comes from a
// V tile staged in LDS by direct buffer->LDS loads and read back with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16).  The head dimension is
// permuted consistently in Q and K (lane half u owns channels u*D/2 ..) so
// every lane loads contiguous bytes.
//
// Every global access goes through a buffer descriptor bounded at the last
// valid row of its (batch, head): rows >= N read as zero and are never
// written, so any N runs on the one build and padding contributes exactly 0.
#include "sol_internal.h"

namespace sol {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLn2 = 0.69314718055994531f;
// The reference row maximum is only moved when a new score exceeds it by more
// than this many powers of two; exp2 values then stay below 2^64, far inside
// float32 and bf16 range.
constexpr float kRescaleSlack = 64.0f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

template <int D>
struct Tile {
    static constexpr int KC = D / 16;             // MFMA k-steps over the head dimension
    static constexpr int DT = D / 32;             // 32-wide output channel tiles
    static constexpr int ROWB = 2 * D;            // bytes of one key row of one head
    static constexpr int CHUNKS = ROWB / 16;      // 16-byte chunks per key row
    static constexpr int VLOADS = 64 * ROWB / 1024;  // direct loads per V tile (16 B per lane)
};

// LDS position of 16-byte chunk `c` of tile row `key`: chunks are XOR-swizzled
// by the row so the transposed reads of 8 consecutive rows spread over all banks.
template <int D>
__device__ __forceinline__ int vchunk(int key, int c) {
    return c ^ ((key * 4) & (Tile<D>::CHUNKS - 1));
}

template <int D, bool DENSE>
__global__ __launch_bounds__(64) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, Geom g, const int16_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, float scale_log2, uint16_t* __restrict__ o,
    float* __restrict__ lse)
{
    using T = Tile<D>;
    __shared__ __attribute__((aligned(1024))) char vbuf0[64 * T::ROWB];
    __shared__ __attribute__((aligned(1024))) char vbuf1[64 * T::ROWB];

    const int work = xcd_remap(blockIdx.x, gridDim.x, g.B * g.H * g.NB);
    if (work < 0) return;
    const int bh = work / g.NB;
    const int qb = work - bh * g.NB;
    const int b = bh / g.H, h = bh - b * g.H;
    const int lane = threadIdx.x;
    const int l32 = lane & 31, u = lane >> 5;

    const int64_t head_off = (int64_t)b * g.sb + (int64_t)h * g.sh;
    const uint32_t rowstride = (uint32_t)(g.sn * 2);
    const uint32_t bound = (uint32_t)(((int64_t)(g.N - 1) * g.sn + D) * 2);
    const __amdgpu_buffer_rsrc_t rq = rsrc(q + head_off, bound);
    const __amdgpu_buffer_rsrc_t rk = rsrc(k + head_off, bound);
    const __amdgpu_buffer_rsrc_t rv = rsrc(v + head_off, bound);

    // ---- Q^T operand, resident for the whole walk
    bf16x8 qop[2][T::KC];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const uint32_t base = (uint32_t)(qb * 64 + 32 * rt + l32) * rowstride + u * D;
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc) qop[rt][kc] = load16(rq, base + 16 * kc);
    }

    // ---- the tile walk: sink tiles, then routed blocks
    const int nsink = DENSE ? g.NB : (g.Ssink + 63) / 64;
    int nlist = 0, first = 0;
    bool straddle_in = false;
    __amdgpu_buffer_rsrc_t rl = rq;
    if (!DENSE) {
        nlist = min(max(cnt[work], 0), g.ncand);
        rl = rsrc(idx + (int64_t)work * g.NB, (uint32_t)nlist * 2);
    }
    // list entries, 64 at a time: lane l holds entry 64 c + l (0 past the end)
    auto list_chunk = [&](int c) -> int {
        return (int)(int16_t)__builtin_amdgcn_raw_buffer_load_b16(rl, (uint32_t)(128 * c + 2 * lane), 0, 0);
    };
    int chunk_id = 0;
    int chunk = 0;
    if (!DENSE && nlist > 0) {
        chunk = list_chunk(0);
        if ((g.S & 63) != 0 && g.S < g.N && __builtin_amdgcn_readlane(chunk, 0) == g.j0) {
            straddle_in = true;
            first = 1;
        }
    }
    const int ntiles = nsink + nlist - first;
    // block of tile t (t must be the current or the next tile)
    auto tile_block = [&](int t) -> int {
        if (DENSE || t < nsink) return t;
        const int e = first + t - nsink;
        if ((e >> 6) != chunk_id) {
            chunk_id = e >> 6;
            chunk = list_chunk(chunk_id);
        }
        return min(max(__builtin_amdgcn_readlane(chunk, e & 63), 0), g.NB - 1);
    };
    auto tile_kmax = [&](int t, int blk) -> int {
        if (DENSE || t >= nsink) return min(64 * blk + 64, g.N);
        if (t < nsink - 1) return 64 * blk + 64;
        return straddle_in ? min(64 * blk + 64, g.N) : g.Ssink;
    };

    // V tile -> LDS by direct loads.  Load n, lane l writes LDS bytes
    // [n * 1024 + 16 l, +16): tile row n * rows_per_load + l / CHUNKS, physical
    // chunk l % CHUNKS.  The row swizzle only depends on the row modulo
    // CHUNKS / 4, which is lane-constant here, so each load needs one VGPR
    // offset per tile plus an SGPR step.
    constexpr int rows_per_load = 1024 / T::ROWB;
    const int vrow = lane / T::CHUNKS;
    const uint32_t v_lane = (uint32_t)vrow * rowstride + 16 * vchunk<D>(vrow, lane % T::CHUNKS);
    auto issue_v = [&](int blk, char* buf) {
        const uint32_t voff = v_lane + (uint32_t)(64 * blk) * rowstride;
#pragma unroll
        for (int n = 0; n < T::VLOADS; ++n)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(buf + n * 1024), 16, voff,
                                                     (uint32_t)(n * rows_per_load) * rowstride, 0, 0);
    };
    // K operand of one 32-key half tile: lane holds key l32, channels u*D/2 ..
    bf16x8 kop[T::KC];
    const uint32_t k_lane = (uint32_t)l32 * rowstride + u * D;
    auto load_k = [&](int blk, int kt) {
        const uint32_t voff = k_lane + (uint32_t)(64 * blk + 32 * kt) * rowstride;
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc)
            kop[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, voff + 16 * kc, 0, 0));
    };
    // transposed-read offsets: row cb + 8 half + 4 u + (lane & 15) / 4 of the
    // tile, channels 32 dt + 16 ((lane >> 4) & 1) + 4 (lane & 3)
    uint32_t v_rd[T::DT];
    {
        const int key = 4 * u + ((lane & 15) >> 2);
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
            const int byte2 = 64 * dt + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
            v_rd[dt] = key * T::ROWB + vchunk<D>(key, byte2 >> 4) * 16 + (byte2 & 15);
        }
    }

    f32x16 oacc[T::DT][2];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) oacc[dt][rt] = f32x16{};
    // mref: per-row reference maximum (log2 units) of the accumulation.  It is
    // fixed by the first half tile and only moved, with O and l rescaled, when
    // a later score exceeds it by more than kRescaleSlack; in between,
    // exp2 values stay below 2^kRescaleSlack.  O and l always share mref, so
    // the final O / l is exact whatever mref is.
    float mref[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.f, 0.f};

    // softmax of one 32-key half tile against mref, then O^T += V^T P^T
    auto finish_half = [&](f32x16 (&s)[2], int kt, const char* cur, bool more) {
        bf16x8 p[2][2];   // [c2][rt]
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float nm = -mref[rt];
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][r], scale_log2, nm));
                s[rt][r] = e;
                acc += e;
            }
            lsum[rt] += acc;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                f32x8 h8;
#pragma unroll
                for (int e = 0; e < 8; ++e) h8[e] = s[rt][8 * c2 + e];
                p[c2][rt] = __builtin_convertvector(h8, bf16x8);
            }
        }
        if (kt == 0) {
            // V(t) must have landed in LDS: wait for all but the loads issued
            // after it (V(t+1) when there is a next tile, and one K half)
            if (more) {
                constexpr int pending = T::VLOADS + T::KC;
                __builtin_amdgcn_s_waitcnt((pending & 15) | ((pending >> 4) << 14) | (7 << 4) | (15 << 8));
            } else {
                constexpr int pending = T::KC;
                __builtin_amdgcn_s_waitcnt((pending & 15) | ((pending >> 4) << 14) | (7 << 4) | (15 << 8));
            }
        }
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            const int cb = 32 * kt + 16 * c2;
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt) {
                bf16x8 vop;
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    // rows cb + 8 half keep the row modulo 4, so the swizzle holds
                    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(cur + v_rd[dt] + (cb + 8 * half) * T::ROWB));
                    const bf16x4 xb = __builtin_bit_cast(bf16x4, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) vop[4 * half + e] = xb[e];
                }
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    oacc[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, p[c2][rt], oacc[dt][rt], 0, 0, 0);
            }
        }
    };

    // walk in 32-key half tiles; step = 2 t + kt
    const int nsteps = 2 * ntiles;
    int blk = ntiles > 0 ? tile_block(0) : 0;
    int nblk = 0;
    if (ntiles > 0) {
        issue_v(blk, vbuf0);
        load_k(blk, 0);
    }
    int step = 0;
    f32x16 s[2];
    float mnew[2];
    while (step < nsteps) {
        bool rescale = false;
        for (; step < nsteps; ++step) {
            const int t = step >> 1, kt = step & 1;
            const bool more = t + 1 < ntiles;
            if (kt == 0) {
                nblk = more ? tile_block(t + 1) : 0;
                if (more) issue_v(nblk, (t & 1) ? vbuf0 : vbuf1);
            }
            // S^T = K Q^T for 32 keys: lane holds rows 32 rt + l32, keys 8 (r/4) + 4 u + r%4
            s[0] = f32x16{};
            s[1] = f32x16{};
#pragma unroll
            for (int kc = 0; kc < T::KC; ++kc)
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
                    s[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kc], qop[rt][kc], s[rt], 0, 0, 0);
            if (kt == 0) load_k(blk, 1);
            else if (more) load_k(nblk, 0);

            const int kmax = tile_kmax(t, blk);
            const int kbase = 64 * blk + 32 * kt;
            if (kmax < kbase + 32) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kbase + 8 * (r / 4) + 4 * u + (r & 3);
                    if (key >= kmax) {
                        s[0][r] = -INFINITY;
                        s[1][r] = -INFINITY;
                    }
                }
            }
            bool need = false;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                float mx = s[rt][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[rt][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                mnew[rt] = mx * scale_log2;
                need |= mnew[rt] > mref[rt] + kRescaleSlack;
            }
            if (__builtin_amdgcn_ballot_w64(need) != 0) {
                rescale = true;
                break;
            }
            finish_half(s, kt, (t & 1) ? vbuf1 : vbuf0, more);
            if (kt == 1) blk = nblk;
        }
        if (rescale) {
            // rare: a score above mref + slack (always at the first half tile)
            const int t = step >> 1, kt = step & 1;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const float m_use = fmaxf(mref[rt], mnew[rt]);
                const float alpha = __builtin_amdgcn_exp2f(mref[rt] - m_use);
                mref[rt] = m_use;
                lsum[rt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < T::DT; ++dt) oacc[dt][rt] *= alpha;
            }
            finish_half(s, kt, (t & 1) ? vbuf1 : vbuf0, t + 1 < ntiles);
            if (kt == 1) blk = nblk;
            ++step;
        }
    }
    const float* mrow = mref;

    // ---- epilogue: normalise, round to bf16, store rows < N only
    const int64_t o_off = (int64_t)b * g.osb + (int64_t)h * g.osh;
    const uint32_t obound = (uint32_t)(((int64_t)(g.N - 1) * g.osn + D) * 2);
    const __amdgpu_buffer_rsrc_t ro = rsrc(o + o_off, obound);
    const uint32_t orow = (uint32_t)(g.osn * 2);
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const float lt = lsum[rt] + __shfl_xor(lsum[rt], 32, 64);
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        const uint32_t row = (uint32_t)(qb * 64 + 32 * rt + l32);
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = oacc[dt][rt][4 * r4 + e] * inv;
                const bf16x4 y = __builtin_convertvector(x, bf16x4);
                const int d0 = 32 * dt + 8 * r4 + 4 * u;
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, y), ro,
                                                      row * orow + 2 * d0, 0, 0);
            }
        if (lse != nullptr && u == 0) {
            const __amdgpu_buffer_rsrc_t rl = rsrc(lse + (int64_t)bh * g.N, (uint32_t)g.N * 4);
            const float val = lt > 0.f ? (mrow[rt] + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rl, row * 4, 0, 0);
        }
    }
}

template <int D, bool DENSE>
hipError_t launch(const Geom& g, const void* q, const void* k, const void* v,
                  const int16_t* idx, const int32_t* cnt, float scale, void* o, float* lse,
                  hipStream_t stream)
{
    const int total = g.B * g.H * g.NB;
    const int grid = round_up(total, kXcds);
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((attn_fwd_kernel<D, DENSE>), dim3(grid), dim3(64), 0, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, idx, cnt,
                       scale_log2, (uint16_t*)o, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const Geom& g, const void* q, const void* k, const void* v,
                       const int16_t* idx, const int32_t* cnt, float scale, void* o,
                       float* lse, bool dense, hipStream_t stream)
{
    if (g.D == 128)
        return dense ? launch<128, true>(g, q, k, v, idx, cnt, scale, o, lse, stream)
                     : launch<128, false>(g, q, k, v, idx, cnt, scale, o, lse, stream);
    return dense ? launch<64, true>(g, q, k, v, idx, cnt, scale, o, lse, stream)
                 : launch<64, false>(g, q, k, v, idx, cnt, scale, o, lse, stream);
}

}  // namespace sol
