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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
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

constexpr int kMaxList = 4096;   // routed blocks per query block (candidate limit)

template <int D, bool DENSE>
__global__ __launch_bounds__(64) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, Geom g, const int16_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ order, float scale_log2,
    uint16_t* __restrict__ o, float* __restrict__ lse)
{
    using T = Tile<D>;
    constexpr int HALF_BYTES = 32 * T::ROWB;         // one 32-key half tile of V
    constexpr int VH = HALF_BYTES / 1024;             // 16-byte loads per lane per half tile
    constexpr int rows_per_load = 1024 / T::ROWB;
    __shared__ __attribute__((aligned(1024))) char vbuf[2][HALF_BYTES];
    // routed list of this query block: round_up(min(ncand, kMaxList), 64)
    // entries of dynamic LDS (sized at launch, so short sequences keep the
    // footprint small and more waves fit on a CU)
    extern __shared__ __attribute__((aligned(16))) int16_t lst[];

    const int work = xcd_remap(blockIdx.x, gridDim.x, g.B * g.H * g.NB);
    if (work < 0) return;
    const int bh = work / g.NB;
    // the rank-th query block of this (batch, head) in the routing schedule
    // (longest list first), or in sequence order without one
    const int rank = work - bh * g.NB;
    const int qb = (DENSE || order == nullptr)
                       ? rank : min(max(order[(int64_t)bh * g.NB + rank], 0), g.NB - 1);
    const int item = bh * g.NB + qb;
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
    // Q is only ever an MFMA source: keep it in AGPRs, which MFMA reads
    // directly, and leave the VGPRs to the scores and the accumulator
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc) asm volatile("" : "+a"(qop[rt][kc]));

    // ---- the tile walk: sink tiles, then routed blocks (list copied to LDS)
    const int nsink = DENSE ? g.NB : (g.Ssink + 63) / 64;
    int nlist = 0, first = 0;
    bool straddle_in = false;
    if (!DENSE) {
        nlist = min(max(cnt[item], 0), min(g.ncand, kMaxList));
        if (nlist > 0) {
            // 2-byte loads: buffer range checks work per dword, so a wider load
            // would drop the last entry of an odd-length list
            const __amdgpu_buffer_rsrc_t rl = rsrc(idx + (int64_t)item * g.NB, (uint32_t)nlist * 2);
            for (int base = 0; base < nlist; base += 64)
                lst[base + lane] = (int16_t)__builtin_amdgcn_raw_buffer_load_b16(
                    rl, (uint32_t)(2 * (base + lane)), 0, 0);
            if ((g.S & 63) != 0 && g.S < g.N && lst[0] == g.j0) {
                straddle_in = true;
                first = 1;
            }
        }
    }
    const int ntiles = nsink + nlist - first;
    auto tile_block = [&](int t) -> int {
        if (DENSE || t < nsink) return t;
        return min(max((int)lst[first + t - nsink], 0), g.NB - 1);
    };
    auto tile_kmax = [&](int t, int blk) -> int {
        if (DENSE || t >= nsink) return min(64 * blk + 64, g.N);
        if (t < nsink - 1) return 64 * blk + 64;
        return straddle_in ? min(64 * blk + 64, g.N) : g.Ssink;
    };

    // V half tile: global -> registers -> LDS.  Load n, lane l covers LDS
    // bytes [n * 1024 + 16 l, +16): half-tile row n * rows_per_load + l / CHUNKS,
    // physical chunk l % CHUNKS.  The row swizzle depends on the row modulo
    // CHUNKS / 4 only, which is lane-constant, so one VGPR offset per half
    // tile plus an SGPR step per load.
    const int vrow = lane / T::CHUNKS;
    const uint32_t v_lane = (uint32_t)vrow * rowstride + 16 * vchunk<D>(vrow, lane % T::CHUNKS);
    // Two register sets each for V and K (half step h uses set h % 2), so
    // both are fetched two half steps ahead of their use.
    uint4 vreg[2][VH];
    auto load_v = [&](int set, int blk, int kt) {
        const uint32_t voff = v_lane + (uint32_t)(64 * blk + 32 * kt) * rowstride;
#pragma unroll
        for (int n = 0; n < VH; ++n)
            vreg[set][n] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                rv, voff, (uint32_t)(n * rows_per_load) * rowstride, 0));
    };
    auto store_v = [&](int set, char* buf) {
#pragma unroll
        for (int n = 0; n < VH; ++n) *(uint4*)(buf + n * 1024 + 16 * lane) = vreg[set][n];
    };
    // K operand of one 32-key half tile: lane holds key l32, channels u*D/2 ..
    bf16x8 kop[2][T::KC];
    const uint32_t k_lane = (uint32_t)l32 * rowstride + u * D;
    auto load_k = [&](int set, int blk, int kt) {
        const uint32_t voff = k_lane + (uint32_t)(64 * blk + 32 * kt) * rowstride;
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc)
            kop[set][kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, voff + 16 * kc, 0, 0));
    };
    // transposed-read offsets in a half-tile buffer: row 16 c2 + 8 half + 4 u +
    // (lane & 15) / 4, channels 32 dt + 16 ((lane >> 4) & 1) + 4 (lane & 3)
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
    // mref: per-row reference maximum (log2 units) of the accumulation, taken
    // from the first half tile.  Scores may exceed it by up to kRescaleSlack
    // (exp2 values then stay below 2^kRescaleSlack).  If one exceeds it by
    // more, the walk restarts from scratch with the larger reference; O and l
    // always share mref, so the final O / l is exact whatever mref is.  The
    // restart keeps O out of any VALU read-modify-write inside the loop nest.
    float mref[2] = {-INFINITY, -INFINITY};
    float lsum[2] = {0.f, 0.f};

    // S^T = K Q^T for the 32 keys whose K sits in kop: lane holds rows
    // 32 rt + l32 and keys 8 (r/4) + 4 u + r%4 of the half tile.
    auto mfma_s = [&](int set, f32x16 (&s)[2]) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                s[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[set][kc], qop[rt][kc], s[rt], 0, 0, 0);
    };
    // keys >= kmax of the half tile at kbase get -inf; row maxima in score units
    auto mask_max = [&](f32x16 (&s)[2], int kbase, int kmax, float (&mx)[2]) {
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
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float m = fmaxf(s[rt][0], s[rt][1]);
#pragma unroll
            for (int r = 2; r < 16; r += 2) m = fmaxf(m, fmaxf(s[rt][r], s[rt][r + 1]));
            mx[rt] = fmaxf(m, __shfl_xor(m, 32, 64));
        }
    };
    auto needs_rescale = [&](const float (&mx)[2]) -> bool {
        const bool need = (mx[0] * scale_log2 > mref[0] + kRescaleSlack) ||
                          (mx[1] * scale_log2 > mref[1] + kRescaleSlack);
        return __builtin_amdgcn_ballot_w64(need) != 0;
    };
    // Row tile rt: p = exp2(s * scale_log2 - mref) as bf16 B operands p[c2][rt];
    // l += sum of the bf16 p (v_dot2 with ones: two keys per instruction, and
    // the same rounded weights that multiply V)
    auto softmax_rt = [&](f32x16 (&s)[2], bf16x8 (&p)[2][2], int rt) {
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        const float nm = -mref[rt];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s[rt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][r], scale_log2, nm));
        float acc = lsum[rt];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            f32x8 h8;
#pragma unroll
            for (int e = 0; e < 8; ++e) h8[e] = s[rt][8 * c2 + e];
            p[c2][rt] = __builtin_convertvector(h8, bf16x8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 pr = {p[c2][rt][2 * e], p[c2][rt][2 * e + 1]};
                acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);
            }
        }
        lsum[rt] = acc;
    };
    // V^T operands of the 32 keys held in the half-tile buffer `cur`
    auto read_v = [&](const char* cur, bf16x8 (&vop)[2][T::DT]) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    // rows 16 c2 + 8 half keep the row modulo 4, so the swizzle holds
                    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(cur + v_rd[dt] + (16 * c2 + 8 * half) * T::ROWB));
                    const bf16x4 xb = __builtin_bit_cast(bf16x4, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) vop[c2][dt][4 * half + e] = xb[e];
                }
    };
    // O^T += V^T P^T for row tile rt over those 32 keys
    auto pv_rt = [&](bf16x8 (&p)[2][2], bf16x8 (&vop)[2][T::DT], int rt) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt)
                oacc[dt][rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[c2][dt], p[c2][rt],
                                                                       oacc[dt][rt], 0, 0, 0);
    };

    // One 32-key half step h = (t, kt).  On entry s_cur holds the masked scores
    // of step h and mx_cur their row maxima; register set (h + 1) % 2 holds K
    // of step h + 1 and V of step h + 1 (both may still be in flight), set
    // h % 2 holds K and V of step h + 2 in flight, and vbuf[kt] holds V of
    // step h.  The S MFMAs of step h + 1 run under this step's softmax, and
    // the masking and maxima of step h + 1 run under this step's P V MFMAs.
    // blk, nblk, nnblk: key blocks of tiles t, t + 1, t + 2 (past the end
    // they repeat a valid block: the prefetches then re-read it, harmlessly,
    // and loads issued on every path keep the compiler's wait counts exact).
    int blk = 0, nblk = 0, nnblk = 0;
    auto half_step = [&](int t, int kt, f32x16 (&s_cur)[2], f32x16 (&s_next)[2],
                         float (&mx_next)[2]) {
        const int nxt = kt ^ 1;           // register set of steps h + 1 and h + 3
        // step h + 3 is (t + 1, 1) when kt = 0 and (t + 2, 0) when kt = 1
        const int blk3 = kt == 0 ? nblk : nnblk;
        // ---- one straight-line scheduling region: the MFMA stream runs
        // S(h+1) then P V(h) back to back while the VALU does softmax(h)
        store_v(nxt, vbuf[nxt]);          // V of step h + 1
        load_v(nxt, blk3, kt ^ 1);        // V of step h + 3
        mfma_s(nxt, s_next);              // harmless extra work after the last step
        load_k(nxt, blk3, kt ^ 1);        // K of step h + 3
        bf16x8 p[2][2];
        bf16x8 vop[2][T::DT];
        softmax_rt(s_cur, p, 0);
        read_v(vbuf[kt], vop);
        pv_rt(p, vop, 0);
        softmax_rt(s_cur, p, 1);
        pv_rt(p, vop, 1);
        __builtin_amdgcn_sched_group_barrier(0x200, VH, 0);        // V stores
        __builtin_amdgcn_sched_group_barrier(0x020, VH, 0);        // V loads
#pragma unroll
        for (int i = 0; i < 2 * T::KC; ++i) {                      // S MFMAs | softmax rt 0
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x020, T::KC, 0);     // K loads
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * T::DT, 0); // V^T reads
#pragma unroll
        for (int i = 0; i < 2 * T::DT; ++i) {                      // P V rt 0 | softmax rt 1
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * T::DT, 0); // P V rt 1
        // ---- after the region (runs under the last MFMAs): the next step's
        // mask and maxima, and the list entry of tile t + 2
        if (kt == 0) {
            nnblk = (t + 2 < ntiles) ? tile_block(t + 2) : nblk;
            mask_max(s_next, 64 * blk + 32, tile_kmax(t, blk), mx_next);
        } else {
            mask_max(s_next, 64 * nblk, tile_kmax(t + 1, nblk), mx_next);
        }
    };

    f32x16 sA[2], sB[2];
    float mxA[2] = {0.f, 0.f}, mxB[2] = {0.f, 0.f};
    for (int pass = 0;; ++pass) {
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) oacc[dt][rt] = f32x16{};
        lsum[0] = 0.f;
        lsum[1] = 0.f;
        if (ntiles == 0) break;
        blk = tile_block(0);
        nblk = ntiles > 1 ? tile_block(1) : blk;
        // steps 0, 1, 2 = (0, 0), (0, 1), (1, 0)
        load_v(0, blk, 0);
        load_k(0, blk, 0);
        load_v(1, blk, 1);
        load_k(1, blk, 1);
        store_v(0, vbuf[0]);
        load_v(0, nblk, 0);
        mfma_s(0, sA);
        load_k(0, nblk, 0);
        mask_max(sA, 64 * blk, tile_kmax(0, blk), mxA);
        if (pass == 0) {
            // every tile holds at least one valid key, so this is finite
            mref[0] = mxA[0] * scale_log2;
            mref[1] = mxA[1] * scale_log2;
        }
        bool restart = false;
        for (int t = 0; t < ntiles; ++t) {
            if (needs_rescale(mxA)) {
                restart = true;
                mref[0] = fmaxf(mref[0], mxA[0] * scale_log2);
                mref[1] = fmaxf(mref[1], mxA[1] * scale_log2);
                break;
            }
            half_step(t, 0, sA, sB, mxB);
            if (needs_rescale(mxB)) {
                restart = true;
                mref[0] = fmaxf(mref[0], mxB[0] * scale_log2);
                mref[1] = fmaxf(mref[1], mxB[1] * scale_log2);
                break;
            }
            half_step(t, 1, sB, sA, mxA);
            blk = nblk;
            nblk = nnblk;
        }
        if (!restart) break;
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
                  const int16_t* idx, const int32_t* cnt, const int32_t* order, float scale,
                  void* o, float* lse, hipStream_t stream)
{
    const int total = g.B * g.H * g.NB;
    const int grid = round_up(total, kXcds);
    const float scale_log2 = scale * 1.4426950408889634f;
    const size_t lds_list = DENSE ? 0 : (size_t)round_up(min(g.ncand, kMaxList), 64) * sizeof(int16_t);
    hipLaunchKernelGGL((attn_fwd_kernel<D, DENSE>), dim3(grid), dim3(64), lds_list, stream,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, idx, cnt,
                       order, scale_log2, (uint16_t*)o, lse);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const Geom& g, const void* q, const void* k, const void* v,
                       const int16_t* idx, const int32_t* cnt, const int32_t* order, float scale,
                       void* o, float* lse, bool dense, hipStream_t stream)
{
    if (g.D == 128)
        return dense ? launch<128, true>(g, q, k, v, idx, cnt, order, scale, o, lse, stream)
                     : launch<128, false>(g, q, k, v, idx, cnt, order, scale, o, lse, stream);
    return dense ? launch<64, true>(g, q, k, v, idx, cnt, order, scale, o, lse, stream)
                 : launch<64, false>(g, q, k, v, idx, cnt, order, scale, o, lse, stream);
}

}  // namespace sol
