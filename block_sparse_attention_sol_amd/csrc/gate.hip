// Sparse-vs-dense correctness gate: error statistics between two attention
// outputs of the same call, over the valid rows.
//
// The tokenfactory.fast post ("Verification that catches what the metrics
// miss") describes Sol-Attn's numerical gate as comparing the sparse output
// with the dense output inside a single attention call; the clawpit.io
// article (paragraph on the Sol-Attn settings) reports it as maximum
// absolute error, mean absolute error and relative L2 error.
//
// stats (float64, device): [0] max |a - b|, [1] sum |a - b|, [2] sum (a - b)^2,
// [3] sum b^2, [4] element count, and the two figures the pages report, [5]
// mean |a - b| = [1] / [4] and [6] relative L2 error sqrt([2] / [3]).  The
// maximum is exact (non-negative floats compared as integers); the sums are
// float64 atomics, so their last bits depend on the order the workgroups
// finish in.
#include "sol_internal.h"

namespace sol {

namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__global__ __launch_bounds__(64) void gate_clear_kernel(double* __restrict__ stats) {
    if (threadIdx.x < 7) stats[threadIdx.x] = 0.0;
}

// mean and relative L2 from the sums (one lane, after gate_kernel)
__global__ __launch_bounds__(64) void gate_finish_kernel(double* __restrict__ stats) {
    if (threadIdx.x == 0) {
        stats[5] = stats[4] > 0.0 ? stats[1] / stats[4] : 0.0;
        stats[6] = stats[3] > 0.0 ? sqrt(stats[2] / stats[3]) : 0.0;
    }
}

// grid: x = row groups of 4 rows, y strides over batch * head; block 256 =
// 4 rows x 64 lanes, each lane covers D / 64 channels of its row
__global__ __launch_bounds__(256) void gate_kernel(const uint16_t* __restrict__ a,
                                                   const uint16_t* __restrict__ b, Geom g,
                                                   double* __restrict__ stats)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    float mx = 0.f;
    double s_abs = 0.0, s_sq = 0.0, s_ref = 0.0;
    int n = 0;
    for (int bh = blockIdx.y; bh < g.B * g.H; bh += gridDim.y) {
        const int bb = bh / g.H, h = bh - bb * g.H;
        const Seq sq = seq_of(g, bb);      // rows of a packed sample end at its own length
        if (row < sq.N) {
            const int64_t off = sq.obase + (int64_t)row * g.osn + (int64_t)h * g.osh;
            for (int d = lane; d < g.D; d += 64) {
                const float x = bf16_to_f32(a[off + d]), y = bf16_to_f32(b[off + d]);
                const float e = fabsf(x - y);
                mx = fmaxf(mx, e);
                s_abs += e;
                s_sq += (double)(x - y) * (double)(x - y);
                s_ref += (double)y * (double)y;
            }
            n += g.D;
        }
    }
    // wave reductions, then one atomic per wave and statistic
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        mx = fmaxf(mx, __shfl_xor(mx, m, 64));
        s_abs += __shfl_xor(s_abs, m, 64);
        s_sq += __shfl_xor(s_sq, m, 64);
        s_ref += __shfl_xor(s_ref, m, 64);
    }
    if (lane == 0 && n > 0) {
        // non-negative floats order like their bit patterns
        atomicMax((unsigned long long*)&stats[0],
                  (unsigned long long)__double_as_longlong((double)mx));
        atomicAdd(&stats[1], s_abs);
        atomicAdd(&stats[2], s_sq);
        atomicAdd(&stats[3], s_ref);
        atomicAdd(&stats[4], (double)n);
    }
}

}  // namespace

hipError_t launch_gate(const Geom& g, const void* a, const void* b, double* stats,
                       hipStream_t stream)
{
    hipLaunchKernelGGL(gate_clear_kernel, dim3(1), dim3(64), 0, stream, stats);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid((g.N + 3) / 4, min(g.B * g.H, 65535));
    hipLaunchKernelGGL(gate_kernel, grid, dim3(256), 0, stream, (const uint16_t*)a,
                       (const uint16_t*)b, g, stats);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gate_finish_kernel, dim3(1), dim3(64), 0, stream, stats);
    return hipGetLastError();
}

}  // namespace sol
