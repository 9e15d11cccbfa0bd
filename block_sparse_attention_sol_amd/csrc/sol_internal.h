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
    const int32_t* cu;       // packed variable-length batch: B + 1 row offsets (device), or null
    int64_t T;               // rows of the packed tensors (with cu only)
};

// Geometry of sample b.  A fixed-length batch gives every sample the call's N
// at offset b * sb.  A packed variable-length batch reads the sample's rows
// [cu[b], cu[b + 1]) from the offsets, clamped so that the sample stays
// inside [0, T) and holds at most N rows: no access can leave the buffers,
// whatever the offsets hold.  The rest follows from the sample's own length
// exactly as on the host: its blocks, sink, first candidate and candidates.
struct Seq {
    int64_t base;    // element offset of the sample's row 0 in Q, K and V
    int64_t obase;   // element offset of the sample's row 0 in O
    int N, NB, Ssink, j0, ncand;
};

__device__ __forceinline__ Seq seq_of(const Geom& g, int b) {
    Seq s;
    int n;
    if (g.cu == nullptr) {
        n = g.N;
        s.base = (int64_t)b * g.sb;
        s.obase = (int64_t)b * g.osb;
    } else {
        const int64_t start = min(max((int64_t)g.cu[b], (int64_t)0), g.T);
        const int64_t end = min(max((int64_t)g.cu[b + 1], start), min(g.T, start + g.N));
        n = (int)(end - start);
        s.base = start * g.sn;
        s.obase = start * g.osn;
    }
    s.N = n;
    s.NB = (n + kBlock - 1) / kBlock;
    s.Ssink = min(g.S, n);
    s.j0 = g.S >= n ? s.NB : g.S / kBlock;
    s.ncand = s.NB - s.j0;
    return s;
}

// Workgroup id -> logical work index, so that consecutive logical indices
// (same head) land on the same XCD and share its L2.  The grid must be a
// multiple of kXcds; ids past `total` return -1.
__device__ __forceinline__ int xcd_remap(int wg, int grid, int total) {
    const int per = grid / kXcds;
    const int logical = (wg % kXcds) * per + wg / kXcds;
    return logical < total ? logical : -1;
}

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Routing launch: K pooling, then scoring with the query blocks pooled on chip
// (+ schedule when order != nullptr).  ws holds room for qbar (unused here),
// kbar, then the scoring workgroups' partial totals.
hipError_t launch_route(const Geom& g, const void* q, const void* k, float scale, float tau,
                        int16_t* idx, int32_t* cnt, int64_t* totals, int32_t* order, float* ws,
                        hipStream_t stream);
size_t route_ws_floats(const Geom& g);

// Routing from block means already in ws (written by launch_qk_norm_rope_pool);
// the partial totals after them are scratch.
hipError_t launch_route_pooled(const Geom& g, float scale, float tau, int16_t* idx, int32_t* cnt,
                               int64_t* totals, int32_t* order, float* ws, hipStream_t stream);

// QK-norm + RoPE producer that also writes the block means into ws (the
// routing workspace layout).  rope_cos / rope_sin may both be null (no RoPE).
hipError_t launch_qk_norm_rope_pool(const Geom& g, const void* q, const void* k,
                                    const float* gamma_q, const float* gamma_k, float eps,
                                    const float* rope_cos, const float* rope_sin, void* q_out,
                                    void* k_out, float* ws, hipStream_t stream);

// Attention launches; order (nullable) is the routing schedule.
hipError_t launch_attn(const Geom& g, const void* q, const void* k, const void* v,
                       const int16_t* idx, const int32_t* cnt, const int32_t* order, float scale,
                       void* o, float* lse, bool dense, hipStream_t stream);

// Sparse-vs-dense gate statistics (float64[5]) of two outputs with O strides.
hipError_t launch_gate(const Geom& g, const void* a, const void* b, double* stats,
                       hipStream_t stream);

}  // namespace sol
