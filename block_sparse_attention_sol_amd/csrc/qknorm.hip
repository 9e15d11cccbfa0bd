// Fused producer for routing on gfx950: per-head RMS normalisation of the
// query and key rows (QK-norm), rotary position embedding (RoPE), the bf16
// outputs that attention reads, and -- in the same pass over the rows -- the
// block means of those outputs that routing scores.
//
// The tokenfactory.fast post ("Custom kernels") lists a fused QK-norm plus
// RoPE kernel among the ops it rewrote; QK-norm and RoPE run on Q and K just
// before attention.  Routing compresses queries and keys into block means
// (clawpit.io article, paragraph on the Sol-Attn settings), so a producer that
// already streams Q and K can emit those means for free and routing need not
// read Q and K again.  The pages define neither operation; the arithmetic
// below (stated in include/sol.h) is the plainest reading, fixed in float32
// order so that the outputs are reproducible bit for bit.
//
// Work decomposition (HBM-bound, like the routing pool): grid x = 64-row
// block, y = 64-lane waves over (head, 8-channel chunk), z = batch x {Q, K};
// one wave per workgroup.  A lane owns 8 channels of one head and walks the
// block's rows in ascending order, with 16-byte loads and stores, and
// accumulates the block mean of its channels in that order.  The D / 8 lanes
// of a head are consecutive and take the rows in groups of D / 8: the group
// is staged in LDS, lane c of the head sums the squares of row c of the group
// in one ascending float32 chain over all D channels, and the resulting scale
// goes back to the head's lanes through LDS.  The pair (2i, 2i + 1) that RoPE
// rotates lies inside one lane's chunk.  The block mean accumulates the
// rounded bf16 outputs in the same ascending order as the routing pool, so
// routing from these means equals routing from the outputs.
#include "sol_internal.h"

namespace sol {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Q and K rows are read once and the outputs written once: non-temporal
// accesses keep the stream from displacing cached lines (6% faster)
__device__ __forceinline__ uint4 load_stream16(const uint16_t* p) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_stream16(uint16_t* p, const uint4& v) {
    __builtin_nontemporal_store((u32x4){v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int D>
__global__ __launch_bounds__(64) void qk_norm_rope_pool_kernel(
    const uint16_t* q, const uint16_t* k, Geom g, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, float eps, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, uint16_t* qo, uint16_t* ko, float* __restrict__ qbar,
    float* __restrict__ kbar)
{
    constexpr int CH = D / 8;                   // lanes per head = rows per group
    constexpr int HPW = 64 / CH;                // heads per wave
    // LDS row of the group: D bf16 plus 16 bytes, so that the 16 lanes reading
    // 16 different rows at the same offset hit distinct banks
    constexpr int ROWB = 2 * D + 16;
    __shared__ __attribute__((aligned(16))) char xs[HPW * CH * ROWB];
    __shared__ __attribute__((aligned(16))) float rs[64];

    const int blk = blockIdx.x;
    const int b = blockIdx.z >> 1;
    const int is_k = blockIdx.z & 1;
    const Seq sq = seq_of(g, b);
    if (blk >= sq.NB) return;                   // past this sample's last block
    const int lane = threadIdx.x;
    const int lane_id = blockIdx.y * 64 + lane;
    // lanes past the last head (whole head groups) compute on head 0 and
    // store nothing
    const bool valid = lane_id < g.H * CH;
    const int h = valid ? lane_id / CH : 0;
    const int hl = lane / CH;                   // head slot within the wave
    const int c = lane % CH;
    const int r0 = blk * kBlock;
    const int r1 = min(r0 + kBlock, sq.N);
    const int pool_from = is_k ? max(r0, g.S) : r0;     // K: routable rows only

    const uint16_t* src = (is_k ? k : q) + sq.base + (int64_t)h * g.sh + c * 8;
    uint16_t* dst = (is_k ? ko : qo) + sq.obase + (int64_t)h * g.osh + c * 8;
    float gm[8];
    {
        const float4* gp = (const float4*)((is_k ? gamma_k : gamma_q) + c * 8);
        const float4 a = gp[0], bb = gp[1];
        gm[0] = a.x; gm[1] = a.y; gm[2] = a.z; gm[3] = a.w;
        gm[4] = bb.x; gm[5] = bb.y; gm[6] = bb.z; gm[7] = bb.w;
    }
    const bool rope = rope_cos != nullptr;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    char* const myrows = xs + hl * CH * ROWB;   // this head's staged rows

    // RoPE tables of 8 rows of the group at a time
    float4 cs[8], sn[8];
    auto load_tables = [&](int t0, int u0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int t = min(t0 + u0 + u, r1 - 1);
            cs[u] = *(const float4*)(rope_cos + (int64_t)t * (D / 2) + c * 4);
            sn[u] = *(const float4*)(rope_sin + (int64_t)t * (D / 2) + c * 4);
        }
    };

    for (int t0 = r0; t0 < r1; t0 += CH) {
        {
            uint4 w[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u)
                w[u] = load_stream16(src + (int64_t)min(t0 + u, r1 - 1) * g.sn);
            if (rope) load_tables(t0, 0);
            // the previous group's LDS reads are done before it is overwritten
            __syncthreads();
#pragma unroll
            for (int u = 0; u < CH; ++u) *(uint4*)(myrows + u * ROWB + c * 16) = w[u];
        }
        __syncthreads();
        // sum of squares of row t0 + c: one running float32 sum over the D
        // channels in ascending order (a bf16 square is exact in float32, so
        // the fused step rounds as the plain one would)
        float ss = 0.f;
        {
            const char* row = myrows + c * ROWB;
#pragma unroll
            for (int kc = 0; kc < CH; ++kc) {
                const uint4 v = *(const uint4*)(row + 16 * kc);
                const uint32_t ws4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = bf_lo(ws4[e]), hi = bf_hi(ws4[e]);
                    ss = __builtin_fmaf(lo, lo, ss);
                    ss = __builtin_fmaf(hi, hi, ss);
                }
            }
        }
        rs[lane] = 1.0f / __builtin_sqrtf(__builtin_fmaf(ss, 1.0f / D, eps));
        __syncthreads();
#pragma unroll
        for (int u0 = 0; u0 < CH; u0 += 8) {
            if (rope && u0 > 0) load_tables(t0, u0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u0 + u;
                if (t >= r1) continue;          // uniform: the whole workgroup shares t
                const uint4 wu = *(const uint4*)(myrows + (u0 + u) * ROWB + c * 16);
                const float x[8] = {bf_lo(wu.x), bf_hi(wu.x), bf_lo(wu.y), bf_hi(wu.y),
                                    bf_lo(wu.z), bf_hi(wu.z), bf_lo(wu.w), bf_hi(wu.w)};
                const float r = rs[hl * CH + u0 + u];
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = (x[e] * r) * gm[e];
                if (rope) {
                    const float co[4] = {cs[u].x, cs[u].y, cs[u].z, cs[u].w};
                    const float si[4] = {sn[u].x, sn[u].y, sn[u].z, sn[u].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float a = y[2 * i], bq = y[2 * i + 1];
                        y[2 * i] = __builtin_fmaf(a, co[i], -(bq * si[i]));
                        y[2 * i + 1] = __builtin_fmaf(a, si[i], bq * co[i]);
                    }
                }
                const bf16x4 lo = __builtin_convertvector((f32x4){y[0], y[1], y[2], y[3]}, bf16x4);
                const bf16x4 hi = __builtin_convertvector((f32x4){y[4], y[5], y[6], y[7]}, bf16x4);
                const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
                const uint4 out = make_uint4(l2.x, l2.y, h2.x, h2.y);
                if (valid) store_stream16(dst + (int64_t)t * g.osn, out);
                if (t >= pool_from) {
                    acc[0] += bf_lo(out.x); acc[1] += bf_hi(out.x);
                    acc[2] += bf_lo(out.y); acc[3] += bf_hi(out.y);
                    acc[4] += bf_lo(out.z); acc[5] += bf_hi(out.z);
                    acc[6] += bf_lo(out.w); acc[7] += bf_hi(out.w);
                }
            }
        }
    }
    if (!valid || (is_k && blk < sq.j0)) return;    // key blocks before j0 are never candidates
    const float rows = (float)(r1 - pool_from);
    const int64_t bh = (int64_t)b * g.H + h;
    float4* pd = !is_k ? (float4*)(qbar + (bh * g.NB + blk) * D + c * 8)
                       : (float4*)(kbar + ((bh * CH + c) * g.NB + blk) * 8);
    pd[0] = make_float4(acc[0] / rows, acc[1] / rows, acc[2] / rows, acc[3] / rows);
    pd[1] = make_float4(acc[4] / rows, acc[5] / rows, acc[6] / rows, acc[7] / rows);
}

}  // namespace

hipError_t launch_qk_norm_rope_pool(const Geom& g, const void* q, const void* k,
                                    const float* gamma_q, const float* gamma_k, float eps,
                                    const float* rope_cos, const float* rope_sin, void* q_out,
                                    void* k_out, float* ws, hipStream_t stream)
{
    const size_t one = ((size_t)g.B * g.H * g.NB * g.D + 63) / 64 * 64;
    float* qbar = ws;
    float* kbar = ws + one;
    const int lanes = g.H * (g.D / 8);
    const dim3 grid(g.NB, (lanes + 63) / 64, g.B * 2);
    if (g.D == 128)
        hipLaunchKernelGGL(qk_norm_rope_pool_kernel<128>, grid, dim3(64), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, g, gamma_q, gamma_k, eps,
                           rope_cos, rope_sin, (uint16_t*)q_out, (uint16_t*)k_out, qbar, kbar);
    else
        hipLaunchKernelGGL(qk_norm_rope_pool_kernel<64>, grid, dim3(64), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, g, gamma_q, gamma_k, eps,
                           rope_cos, rope_sin, (uint16_t*)q_out, (uint16_t*)k_out, qbar, kbar);
    return hipGetLastError();
}

}  // namespace sol
