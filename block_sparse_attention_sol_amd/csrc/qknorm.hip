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
// block, y = groups of 256 lanes over (head, 8-channel chunk), z = batch x
// {Q, K}.  A lane owns 8 channels of one head and walks the block's rows in
// ascending order: the D / 8 lanes of one head are consecutive, aligned to the
// 16-lane DPP rows, so a row's sum of squares is one DPP tree; the pair
// (2i, 2i + 1) that RoPE rotates lies inside one lane's chunk.  The block mean
// accumulates the rounded bf16 outputs in the same ascending order as the
// routing pool, so routing from these means equals routing from the outputs.
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum of the per-lane partials p_c of one head's CH = D / 8 consecutive lanes
// as the balanced binary tree over c in index order, ((p0 + p1) + (p2 + p3))
// + ..., identical in every lane of the group: each step adds the partner
// group's partial sum, and float addition is commutative, so both partners
// get the same bits.
template <int CH>
__device__ __forceinline__ float head_sum(float v) {
    v += dpp<0xB1>(v);                       // lane ^ 1   (quad_perm [1,0,3,2])
    v += dpp<0x4E>(v);                       // lane ^ 2   (quad_perm [2,3,0,1])
    v += dpp<0x141>(v);                      // other quad of 8 (row_half_mirror)
    if constexpr (CH == 16) v += dpp<0x140>(v);   // other half of 16 (row_mirror)
    return v;
}

template <int D>
__global__ __launch_bounds__(256) void qk_norm_rope_pool_kernel(
    const uint16_t* q, const uint16_t* k, Geom g, const float* __restrict__ gamma_q,
    const float* __restrict__ gamma_k, float eps, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, uint16_t* qo, uint16_t* ko, float* __restrict__ qbar,
    float* __restrict__ kbar)
{
    constexpr int CH = D / 8;                   // lanes per head
    const int blk = blockIdx.x;
    const int b = blockIdx.z >> 1;
    const int is_k = blockIdx.z & 1;
    const Seq sq = seq_of(g, b);
    if (blk >= sq.NB) return;                   // past this sample's last block
    const int lane_id = blockIdx.y * 256 + threadIdx.x;
    // lanes past the last head (whole head groups) compute on head 0 and
    // store nothing, so every DPP step reads an active lane
    const bool valid = lane_id < g.H * CH;
    const int h = valid ? lane_id / CH : 0;
    const int c = lane_id % CH;
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

    constexpr int AHEAD = 8;                    // rows whose loads are in flight together
    for (int t0 = r0; t0 < r1; t0 += AHEAD) {
        uint4 w[AHEAD];
        float4 cs[AHEAD], sn[AHEAD];
#pragma unroll
        for (int u = 0; u < AHEAD; ++u) {
            const int t = min(t0 + u, r1 - 1);
            w[u] = load_stream16(src + (int64_t)t * g.sn);
            if (rope) {
                cs[u] = *(const float4*)(rope_cos + (int64_t)t * (D / 2) + c * 4);
                sn[u] = *(const float4*)(rope_sin + (int64_t)t * (D / 2) + c * 4);
            }
        }
#pragma unroll
        for (int u = 0; u < AHEAD; ++u) {
            const int t = t0 + u;
            if (t >= r1) break;                 // uniform: the whole workgroup shares t
            const float x[8] = {bf_lo(w[u].x), bf_hi(w[u].x), bf_lo(w[u].y), bf_hi(w[u].y),
                                bf_lo(w[u].z), bf_hi(w[u].z), bf_lo(w[u].w), bf_hi(w[u].w)};
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) p = __builtin_fmaf(x[e], x[e], p);
            const float ss = head_sum<CH>(p);
            const float r = 1.0f / __builtin_sqrtf(__builtin_fmaf(ss, 1.0f / D, eps));
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
    const dim3 grid(g.NB, (lanes + 255) / 256, g.B * 2);
    if (g.D == 128)
        hipLaunchKernelGGL(qk_norm_rope_pool_kernel<128>, grid, dim3(256), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, g, gamma_q, gamma_k, eps,
                           rope_cos, rope_sin, (uint16_t*)q_out, (uint16_t*)k_out, qbar, kbar);
    else
        hipLaunchKernelGGL(qk_norm_rope_pool_kernel<64>, grid, dim3(256), 0, stream,
                           (const uint16_t*)q, (const uint16_t*)k, g, gamma_q, gamma_k, eps,
                           rope_cos, rope_sin, (uint16_t*)q_out, (uint16_t*)k_out, qbar, kbar);
    return hipGetLastError();
}

}  // namespace sol
