// Internal declarations shared by the HIP translation units of libsol.
// Not part of the C ABI (include/sol.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sol {

constexpr int kBlock = 64;       // token block (routing and tile granularity)
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dispatched round-robin

// Geometry of one call, computed on the host.
struct Geom {
    int B, N, H, D;
    int NB;        // ceil(N / 64)
    int S;         // sink length as given
    int Ssink;     // min(S, N)
    int j0;        // first candidate key block (NB if none)
    int ncand;     // NB - j0
    int64_t sb, sn, sh;      // Q/K/V element strides
    int64_t osb, osn, osh;   // O element strides
};

// Workgroup id -> logical work index, so that consecutive logical indices
// (same head) land on the same XCD and share its L2.  The grid must be a
// multiple of kXcds; ids past `total` return -1.
__device__ __forceinline__ int xcd_remap(int wg, int grid, int total) {
    const int per = grid / kXcds;
    const int logical = (wg % kXcds) * per + wg / kXcds;
    return logical < total ? logical : -1;
}

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Routing launch: pool + score/select (+ schedule when order != nullptr).
// ws holds qbar then kbar.
hipError_t launch_route(const Geom& g, const void* q, const void* k, float scale, float tau,
                        int16_t* idx, int32_t* cnt, int64_t* totals, int32_t* order, float* ws,
                        hipStream_t stream);
size_t route_ws_floats(const Geom& g);

// Attention launches; order (nullable) is the routing schedule.
hipError_t launch_attn(const Geom& g, const void* q, const void* k, const void* v,
                       const int16_t* idx, const int32_t* cnt, const int32_t* order, float scale,
                       void* o, float* lse, bool dense, hipStream_t stream);

// Sparse-vs-dense gate statistics (float64[5]) of two outputs with O strides.
hipError_t launch_gate(const Geom& g, const void* a, const void* b, double* stats,
                       hipStream_t stream);

}  // namespace sol
