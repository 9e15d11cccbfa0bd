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
// Work decomposition: one workgroup of two waves per (batch, head, query
// block); wave w owns query rows 32 w .. 32 w + 31 of the block (the dense
// walk, the same for every block, takes two blocks and four waves).  The walk
// goes in 32-key half steps.  Both waves fetch the K and V half tile of the
// next step straight from global memory into LDS (buffer loads with the LDS
// destination, 16 bytes per lane) while they compute the current one, so the
// two waves share every K/V byte and a wave needs no staging registers; at
// about 200 VGPRs per wave two waves fit on each SIMD, and the SIMD overlaps
// one wave's softmax VALU work with the other's MFMA work.
//
// Per half step a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = K from LDS, B = Q^T held in registers for the whole walk), so each lane
// holds 16 scores of one query row and a row's statistics need a single
// cross-lane step (lane l and l ^ 32 share a row).  Then O^T += V^T P^T: P is
// rounded to bf16 in place as the B operand, and V^T comes from the LDS half
// tile through the gfx950 transposing read (ds_read_b64_tr_b16).  The head
// dimension is permuted consistently in Q and K (lane half u owns channels
// u*D/2 ..) so that every lane reads contiguous 16-byte chunks.
//
// Every global access goes through a buffer descriptor bounded at the last
// valid row of its (batch, head), with the whole offset in the VGPR operand:
// rows >= N read as zero and are never written, so any N runs on the one
// build and padding contributes exactly 0.  In a packed variable-length batch
// each sample brings its own row offset and length N; the grid is sized by
// the longest sample, and workgroups past a shorter sample's last block exit
// at once.
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
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

constexpr float kLn2 = 0.69314718055994531f;
// A row's reference maximum (log2 units) only moves, with O and l rescaled,
// when a new score exceeds it by more than this many powers of two; between
// moves the exp2 weights stay below 2^kRescaleSlack, far inside float32 and
// bf16 range.  Moves are rare, so the rescale sits off the main path.
constexpr float kRescaleSlack = 16.0f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS: lane l writes
// lds + 16 l (the LDS base must be wave-uniform)
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, char* lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(0), other counters untouched (gfx9 encoding)
__device__ __forceinline__ void wait_vmem_all() {
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
}

template <int D, int NW = 2>
struct Tile {
    static constexpr int KC = D / 16;             // MFMA k-steps over the head dimension
    static constexpr int DT = D / 32;             // 32-wide output channel tiles
    static constexpr int ROWB = 2 * D;            // bytes of one key row of one head
    static constexpr int CHUNKS = ROWB / 16;      // 16-byte chunks per key row
    static constexpr int HB = 32 * ROWB;          // bytes of a 32-key half tile (K or V)
    static constexpr int LOADS = HB / 1024;       // 1 KB wave loads per half tile
    static constexpr int WLOADS = LOADS / NW;     // ... issued by each of the NW waves
    static constexpr int RPL = 1024 / ROWB;       // key rows per 1 KB load
};

// LDS position of 16-byte chunk `c` of K row `key`: XOR-swizzled by the row so
// that the 16 lanes of one read phase (rows r .. r+15, same chunk) hit
// distinct banks.
template <int D>
__device__ __forceinline__ int kchunk(int key, int c) {
    return c ^ (key & (Tile<D>::CHUNKS - 1));
}

// LDS position of 16-byte chunk `c` of V row `key`: swizzled so that the
// transposed reads of 8 consecutive rows spread over all banks.
template <int D>
__device__ __forceinline__ int vchunk(int key, int c) {
    return c ^ ((key * 4) & (Tile<D>::CHUNKS - 1));
}

constexpr int kMaxList = 4096;   // routed blocks per query block (candidate limit)

template <int D, bool DENSE>
__global__ __launch_bounds__(DENSE ? 256 : 128) void
attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, Geom g, const int16_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ order, float scale_log2,
    uint16_t* __restrict__ o, float* __restrict__ lse)
{
    // query blocks per workgroup: the dense walk is the same for every query
    // block, so two blocks (128 rows, four waves) share each fetched tile;
    // routed walks differ per block, so they get one block (two waves) each
    constexpr int NQ = DENSE ? 2 : 1;
    constexpr int NW = 2 * NQ;
    using T = Tile<D, NW>;
    __shared__ __attribute__((aligned(1024))) char kbuf[2][T::HB];
    __shared__ __attribute__((aligned(1024))) char vbuf[2][T::HB];
    // routed list of this query block: round_up(min(ncand, kMaxList), 128)
    // entries of dynamic LDS, sized at launch
    extern __shared__ __attribute__((aligned(16))) int16_t lst[];

    const int nbw = (g.NB + NQ - 1) / NQ;                  // workgroups per (batch, head)
    const int work = xcd_remap(blockIdx.x, gridDim.x, g.B * g.H * nbw);
    if (work < 0) return;
    const int bh = work / nbw;
    const int b = bh / g.H, h = bh - b * g.H;
    // this sample's length and blocks (all equal unless the batch is packed)
    const Seq sq = seq_of(g, b);
    // the rank-th query block of this (batch, head) in the routing schedule
    // (longest list first), or in sequence order without one; ranks past the
    // sample's own blocks have no work
    const int rank = work - bh * nbw;
    if (NQ * rank >= sq.NB) return;
    const int qb = DENSE ? NQ * rank
                 : order == nullptr ? rank
                                    : min(max(order[(int64_t)bh * g.NB + rank], 0), sq.NB - 1);
    const int item = bh * g.NB + qb;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // wave w owns rows 32 (w & 1) .. +31 of query block qb + (w >> 1); past the
    // last block (odd NB, dense) it repeats the last block, whose rows it then
    // writes with the same values as its partner waves
    const int qrow0 = min(qb + (wave >> 1), sq.NB - 1) * 64 + 32 * (wave & 1);
    const int lane = tid & 63;
    const int l32 = lane & 31, u = lane >> 5;

    const int64_t head_off = sq.base + (int64_t)h * g.sh;
    const uint32_t rowstride = (uint32_t)(g.sn * 2);
    const uint32_t bound = (uint32_t)(((int64_t)(sq.N - 1) * g.sn + D) * 2);
    const __amdgpu_buffer_rsrc_t rq = rsrc(q + head_off, bound);
    const __amdgpu_buffer_rsrc_t rk = rsrc(k + head_off, bound);
    const __amdgpu_buffer_rsrc_t rv = rsrc(v + head_off, bound);

    // ---- Q^T operand of this wave's 32 rows, resident for the whole walk
    bf16x8 qop[T::KC];
    {
        const uint32_t base = (uint32_t)(qrow0 + l32) * rowstride + u * D;
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc) qop[kc] = load16(rq, base + 16 * kc);
    }

    // ---- the tile walk: sink tiles, then routed blocks (list copied to LDS)
    const int nsink = DENSE ? sq.NB : (sq.Ssink + 63) / 64;
    int nlist = 0;
    if (!DENSE) {
        nlist = min(max(cnt[item], 0), min(sq.ncand, kMaxList));
        if (nlist > 0) {
            // 2-byte loads: buffer range checks work per dword, so a wider load
            // would drop the last entry of an odd-length list
            const __amdgpu_buffer_rsrc_t rl = rsrc(idx + (int64_t)item * g.NB, (uint32_t)nlist * 2);
            for (int base = 0; base < nlist; base += 64 * NW)
                lst[base + tid] = (int16_t)__builtin_amdgcn_raw_buffer_load_b16(
                    rl, (uint32_t)(2 * (base + tid)), 0, 0);
        }
    }
    __syncthreads();
    int first = 0;
    bool straddle_in = false;
    if (!DENSE && nlist > 0 && (g.S & 63) != 0 && g.S < sq.N && lst[0] == sq.j0) {
        // the straddle block's routable keys join its (masked) sink tile
        straddle_in = true;
        first = 1;
    }
    const int ntiles = nsink + nlist - first;
    auto tile_block = [&](int t) -> int {
        if (DENSE || t < nsink) return t;
        return min(max((int)lst[first + t - nsink], 0), sq.NB - 1);
    };
    auto tile_kmax = [&](int t, int blk) -> int {
        if (DENSE || t >= nsink) return min(64 * blk + 64, sq.N);
        if (t < nsink - 1) return 64 * blk + 64;
        return straddle_in ? min(64 * blk + 64, sq.N) : sq.Ssink;
    };

    // ---- global -> LDS half-tile loads.  Wave load n (this wave issues
    // n = wave * WLOADS + m) fills LDS bytes [n * 1024, +1024): lane l writes
    // half-tile row n * RPL + l / CHUNKS at physical chunk l % CHUNKS, so it
    // fetches the logical chunk that the swizzle puts there.  The lane offsets
    // depend only on the wave, m and the lane, so they are precomputed per m.
    uint32_t k_lane[T::WLOADS], v_lane;
    {
        const int r = lane / T::CHUNKS, pc = lane % T::CHUNKS;
#pragma unroll
        for (int m = 0; m < T::WLOADS; ++m) {
            const int row = (wave * T::WLOADS + m) * T::RPL + r;
            k_lane[m] = (uint32_t)r * rowstride + 16 * kchunk<D>(row, pc);
        }
        v_lane = (uint32_t)r * rowstride + 16 * vchunk<D>(r, pc);
    }
    // key rows [64 blk + 32 half, +32) of K or V into the LDS half tile dst
    auto issue_k = [&](char* dst, int blk, int half) {
        const uint32_t row0 = (uint32_t)(64 * blk + 32 * half + wave * T::WLOADS * T::RPL);
#pragma unroll
        for (int m = 0; m < T::WLOADS; ++m)
            load_lds16(rk, dst + (wave * T::WLOADS + m) * 1024,
                       k_lane[m] + (row0 + (uint32_t)(m * T::RPL)) * rowstride);
    };
    auto issue_v = [&](char* dst, int blk, int half) {
        const uint32_t row0 = (uint32_t)(64 * blk + 32 * half + wave * T::WLOADS * T::RPL);
#pragma unroll
        for (int m = 0; m < T::WLOADS; ++m)
            load_lds16(rv, dst + (wave * T::WLOADS + m) * 1024,
                       v_lane + (row0 + (uint32_t)(m * T::RPL)) * rowstride);
    };

    // K operand reads: lane reads row l32, logical chunk u*CHUNKS/2 + kc
    uint32_t k_rd[T::KC];
#pragma unroll
    for (int kc = 0; kc < T::KC; ++kc)
        k_rd[kc] = l32 * T::ROWB + 16 * kchunk<D>(l32, u * (T::CHUNKS / 2) + kc);
    // V^T transposed-read offsets: row 16 c2 + 8 half + 4 u + (lane & 15) / 4,
    // channels 32 dt + 16 ((lane >> 4) & 1) + 4 (lane & 3)
    uint32_t v_rd[T::DT];
    {
        const int key = 4 * u + ((lane & 15) >> 2);
#pragma unroll
        for (int dt = 0; dt < T::DT; ++dt) {
            const int byte2 = 64 * dt + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
            v_rd[dt] = key * T::ROWB + vchunk<D>(key, byte2 >> 4) * 16 + (byte2 & 15);
        }
    }
    auto read_k = [&](const char* src, bf16x8 (&kop)[T::KC]) {
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc)
            kop[kc] = __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(src + k_rd[kc]));
    };
    auto read_v = [&](const char* src, bf16x8 (&vop)[2][T::DT]) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    // rows 16 c2 + 8 hf keep the row modulo 4, so the swizzle holds
                    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4*)(src + v_rd[dt] + (16 * c2 + 8 * hf) * T::ROWB));
                    const bf16x4 xb = __builtin_bit_cast(bf16x4, x);
#pragma unroll
                    for (int e = 0; e < 4; ++e) vop[c2][dt][4 * hf + e] = xb[e];
                }
    };

    f32x16 oacc[T::DT];
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt) oacc[dt] = f32x16{};
    float mref = -INFINITY;   // row reference maximum, log2 units
    float lsum = 0.f;         // this lane's half of the row's weight sum
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // S^T = K Q^T for one half tile: lane holds row 32 wave + l32, keys
    // 8 (r/4) + 4 u + r%4 of the half tile
    auto mfma_s = [&](const bf16x8 (&kop)[T::KC]) -> f32x16 {
        f32x16 s = f32x16{};
#pragma unroll
        for (int kc = 0; kc < T::KC; ++kc)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kc], qop[kc], s, 0, 0, 0);
        return s;
    };
    // keys >= kmax of the half tile starting at key kbase get -inf
    auto mask = [&](f32x16& s, int kbase, int kmax) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kbase + 8 * (r / 4) + 4 * u + (r & 3);
            if (key >= kmax) s[r] = -INFINITY;
        }
    };
    // row maximum in log2 units; lanes l and l ^ 32 hold the two halves of a row
    auto row_max = [&](const f32x16& s) -> float {
        float m = fmaxf(s[0], s[1]);
#pragma unroll
        for (int r = 2; r < 16; r += 2) m = fmaxf(m, fmaxf(s[r], s[r + 1]));
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                         false, false);
        return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * scale_log2;
    };
    // move the reference maximum when a row's new maximum exceeds it by more
    // than kRescaleSlack (rare: a uniform branch off the main path)
    auto rescale = [&](float mx) {
        if (__builtin_amdgcn_ballot_w64(mx > mref + kRescaleSlack) != 0) {
            const float mnew = fmaxf(mref, mx);
            const float f = __builtin_amdgcn_exp2f(mref - mnew);
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt) oacc[dt] *= f;
            lsum *= f;
            mref = mnew;
        }
    };
    // p = exp2(s * scale_log2 - mref) rounded to bf16; l += the same rounded
    // weights that multiply V (v_dot2 with ones, two per instruction)
    auto softmax = [&](const f32x16& s, bf16x8 (&p)[2]) {
        const float nm = -mref;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            f32x8 h8;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                h8[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * c2 + e], scale_log2, nm));
            p[c2] = __builtin_convertvector(h8, bf16x8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 pr = {p[c2][2 * e], p[c2][2 * e + 1]};
                lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
            }
        }
        // keep the row-sum chain here, in the shadow of this half step's
        // MFMAs: left alone, the compiler sinks it below the mask and rescale
        // branches, where it runs as a serial chain with the MFMA unit idle
        asm volatile("" : "+v"(lsum));
    };
    // O^T += V^T P^T
    auto pv = [&](const bf16x8 (&vop)[2][T::DT], const bf16x8 (&p)[2]) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
            for (int dt = 0; dt < T::DT; ++dt)
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[c2][dt], p[c2], oacc[dt], 0, 0, 0);
    };
    // LDS reads complete in issue order (lgkmcnt), so the K operand reads go
    // out first and alone: queued behind the slower transposed V reads they
    // would hold back the S MFMAs of the whole half step
    auto k_first = [&]() { __builtin_amdgcn_sched_barrier(0); };
    // instruction order of one half step: LDS operand reads, the next loads,
    // then the S MFMAs of the next half step interleaved with this half
    // step's softmax, then the P V MFMAs interleaved with the rest of it and
    // the next row maxima.  At D = 128 four VALU instructions go with every
    // MFMA of both phases (measured against 6 per S MFMA and 2 per P V MFMA,
    // outputs identical: 0.2-0.7% faster sparse, 1.0-1.3% faster dense; 5/3,
    // 3/5, 3/4 and 7/2 were slower on one path or both).
    constexpr int S_VALU = D == 128 ? 4 : 48 / T::KC;
    constexpr int PV_VALU = D == 128 ? 4 : 2;
    auto schedule = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * T::DT, 0);           // V^T LDS reads
        __builtin_amdgcn_sched_group_barrier(0x020, 2 * T::WLOADS, 0);       // loads to LDS
#pragma unroll
        for (int i = 0; i < T::KC; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, S_VALU, 0);
        }
#pragma unroll
        for (int i = 0; i < 2 * T::DT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, PV_VALU, 0);
        }
    };

    // ---- the walk, software-pipelined in 32-key half steps h = 2 t + kt.
    // Half step h computes P V of h and S of h + 1; LDS holds K(h + 1) and
    // V(h) when it starts, and it loads K(h + 2) and V(h + 1) into the
    // buffers that K(h) and V(h - 1) left.  Past the end of the walk the
    // loads repeat the last block (harmless: nothing reads the result).
    if (ntiles > 0) {
        int cblk = tile_block(0);
        issue_k(kbuf[0], cblk, 0);
        issue_v(vbuf[0], cblk, 0);
        issue_k(kbuf[1], cblk, 1);
        wait_vmem_all();
        __syncthreads();
        f32x16 s_cur;
        {
            bf16x8 kop[T::KC];
            read_k(kbuf[0], kop);
            s_cur = mfma_s(kop);
            const int km = tile_kmax(0, cblk);
            if (km < 64 * cblk + 32) mask(s_cur, 64 * cblk, km);
            rescale(row_max(s_cur));
        }
        for (int t = 0; t < ntiles; ++t) {
            // block of tile t + 1 (LDS list read before the wait, which any
            // LDS read would have to take anyway)
            const int nblk = tile_block(min(t + 1, ntiles - 1));
            bf16x8 kop[T::KC];
            bf16x8 vop[2][T::DT];
            bf16x8 p[2];
            // -- half 0 of tile t: P V(t, 0), S(t, 1)
            wait_vmem_all();
            __syncthreads();
            read_k(kbuf[1], kop);            // K(t, 1)
            k_first();
            read_v(vbuf[0], vop);            // V(t, 0)
            issue_k(kbuf[0], nblk, 0);       // K(t + 1, 0)
            issue_v(vbuf[1], cblk, 1);       // V(t, 1)
            f32x16 s_nxt = mfma_s(kop);
            softmax(s_cur, p);
            pv(vop, p);
            float mx = row_max(s_nxt);
            schedule();
            {
                const int km = tile_kmax(t, cblk);
                if (km < 64 * cblk + 64) {
                    mask(s_nxt, 64 * cblk + 32, km);
                    mx = row_max(s_nxt);
                }
            }
            rescale(mx);
            s_cur = s_nxt;
            // -- half 1 of tile t: P V(t, 1), S(t + 1, 0)
            wait_vmem_all();
            __syncthreads();
            read_k(kbuf[0], kop);            // K(t + 1, 0)
            k_first();
            read_v(vbuf[1], vop);            // V(t, 1)
            issue_k(kbuf[1], nblk, 1);       // K(t + 1, 1)
            issue_v(vbuf[0], nblk, 0);       // V(t + 1, 0)
            s_nxt = mfma_s(kop);
            softmax(s_cur, p);
            pv(vop, p);
            mx = row_max(s_nxt);
            schedule();
            if (t + 1 < ntiles) {
                const int km = tile_kmax(t + 1, nblk);
                if (km < 64 * nblk + 32) {
                    mask(s_nxt, 64 * nblk, km);
                    mx = row_max(s_nxt);
                }
                rescale(mx);
            }
            s_cur = s_nxt;
            cblk = nblk;
        }
    }

    // ---- epilogue: normalise, round to bf16, store rows < N only
    const int64_t o_off = sq.obase + (int64_t)h * g.osh;
    const uint32_t obound = (uint32_t)(((int64_t)(sq.N - 1) * g.osn + D) * 2);
    const __amdgpu_buffer_rsrc_t ro = rsrc(o + o_off, obound);
    const uint32_t orow = (uint32_t)(g.osn * 2);
    const auto lsw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum),
                                                      false, false);
    const float lt = __uint_as_float(lsw[0]) + __uint_as_float(lsw[1]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const uint32_t row = (uint32_t)(qrow0 + l32);
#pragma unroll
    for (int dt = 0; dt < T::DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = oacc[dt][4 * r4 + e] * inv;
            const bf16x4 y = __builtin_convertvector(x, bf16x4);
            const int d0 = 32 * dt + 8 * r4 + 4 * u;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, y), ro,
                                                  row * orow + 2 * d0, 0, 0);
        }
    if (lse != nullptr && u == 0) {
        const __amdgpu_buffer_rsrc_t rl = rsrc(lse + (int64_t)bh * g.N, (uint32_t)sq.N * 4);
        const float val = lt > 0.f ? (mref + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, val), rl, row * 4, 0, 0);
    }
}

template <int D, bool DENSE>
hipError_t launch(const Geom& g, const void* q, const void* k, const void* v,
                  const int16_t* idx, const int32_t* cnt, const int32_t* order, float scale,
                  void* o, float* lse, hipStream_t stream)
{
    constexpr int NQ = DENSE ? 2 : 1;
    const int total = g.B * g.H * ((g.NB + NQ - 1) / NQ);
    const int grid = round_up(total, kXcds);
    const float scale_log2 = scale * 1.4426950408889634f;
    const size_t lds_list = DENSE ? 0 : (size_t)round_up(min(g.ncand, kMaxList), 128) * sizeof(int16_t);
    hipLaunchKernelGGL((attn_fwd_kernel<D, DENSE>), dim3(grid), dim3(64 * 2 * NQ), lds_list, stream,
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
