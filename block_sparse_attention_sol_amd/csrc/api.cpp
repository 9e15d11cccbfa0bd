// C ABI of libsol (declared in include/sol.h): argument checks on the host,
// call geometry, and kernel launches on the caller's stream.  No allocation,
// no synchronisation, no printing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "sol.h"
#include "sol_internal.h"

namespace {

constexpr int64_t kMaxCandidates = 4096;   // candidate key blocks per row (routing lists)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every entry point; fills the geometry on success.
sol_status check_desc(const sol_desc* d, int32_t sink_len, sol::Geom* g) {
    if (d == nullptr) return SOL_ERR_ARG;
    if (d->B <= 0 || d->N <= 0 || d->H <= 0 || d->D <= 0 || sink_len < 0) return SOL_ERR_ARG;
    if (d->D != 64 && d->D != 128) return SOL_ERR_UNSUPPORTED;
    if (d->qkv_sb < 0 || d->qkv_sn <= 0 || d->qkv_sh < 0 || d->o_sb < 0 || d->o_sn <= 0 || d->o_sh < 0)
        return SOL_ERR_ARG;
    // rows must be 16-byte aligned: every stride a multiple of 8 bf16 elements
    if ((d->qkv_sb | d->qkv_sn | d->qkv_sh | d->o_sb | d->o_sn | d->o_sh) & 7) return SOL_ERR_ALIGN;
    const int64_t NB = (d->N + sol::kBlock - 1) / sol::kBlock;
    // work items index with 32-bit ints
    if ((int64_t)d->B * d->H * NB >= (int64_t)1 << 30) return SOL_ERR_UNSUPPORTED;
    // per-(batch, head) buffer windows are addressed with 32-bit byte offsets,
    // including the padded tail rows up to 64 * NB
    const int64_t span_in = ((64 * NB - 1) * d->qkv_sn + d->D) * 2;
    const int64_t span_out = ((64 * NB - 1) * d->o_sn + d->D) * 2;
    if (span_in >= ((int64_t)1 << 32) || span_out >= ((int64_t)1 << 32)) return SOL_ERR_UNSUPPORTED;
    if ((int64_t)d->H * d->N >= ((int64_t)1 << 30)) return SOL_ERR_UNSUPPORTED;
    if (d->cu_seqlens != nullptr) {
        // packed variable-length batch: rows are addressed through the offsets
        if (d->qkv_sb != 0 || d->o_sb != 0 || d->total_rows < 0) return SOL_ERR_ARG;
        if (d->total_rows > INT32_MAX) return SOL_ERR_UNSUPPORTED;
        if ((reinterpret_cast<uintptr_t>(d->cu_seqlens) & 3u) != 0) return SOL_ERR_ALIGN;
    }

    g->B = d->B;
    g->N = d->N;
    g->H = d->H;
    g->D = d->D;
    g->NB = (int)NB;
    g->S = sink_len;
    g->Ssink = sink_len < d->N ? sink_len : d->N;
    g->j0 = sink_len >= d->N ? (int)NB : sink_len / sol::kBlock;
    g->ncand = g->NB - g->j0;
    g->sb = d->qkv_sb;
    g->sn = d->qkv_sn;
    g->sh = d->qkv_sh;
    g->osb = d->o_sb;
    g->osn = d->o_sn;
    g->osh = d->o_sh;
    g->cu = d->cu_seqlens;
    g->T = d->cu_seqlens != nullptr ? d->total_rows : 0;
    return SOL_OK;
}

bool same_io_strides(const sol_desc* d) {
    return d->qkv_sb == d->o_sb && d->qkv_sn == d->o_sn && d->qkv_sh == d->o_sh;
}

float resolve_scale(float scale, int D) {
    return scale == 0.0f ? (float)(1.0 / std::sqrt((double)D)) : scale;
}

}  // namespace

extern "C" {

int32_t sol_num_blocks(int32_t N) { return N <= 0 ? 0 : (N + sol::kBlock - 1) / sol::kBlock; }

size_t sol_route_workspace_bytes(const sol_desc* desc) {
    sol::Geom g;
    if (check_desc(desc, 0, &g) != SOL_OK) return 0;
    return sol::route_ws_floats(g) * sizeof(float) + 256;
}

sol_status sol_route(const void* q, const void* k, const sol_desc* desc, float tau,
                     int32_t sink_len, float scale, int16_t* blk_idx, int32_t* blk_cnt,
                     int64_t* totals, int32_t* order, void* workspace, size_t ws_bytes,
                     void* stream) {
    sol::Geom g;
    const sol_status st = check_desc(desc, sink_len, &g);
    if (st != SOL_OK) return st;
    if (q == nullptr || k == nullptr || blk_idx == nullptr || blk_cnt == nullptr || totals == nullptr)
        return SOL_ERR_ARG;
    if (std::isnan(tau) || tau < 0.0f || std::isnan(scale) || scale < 0.0f || std::isinf(scale))
        return SOL_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(totals) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(blk_cnt) & 3u) != 0 || (reinterpret_cast<uintptr_t>(blk_idx) & 1u) != 0 ||
        (reinterpret_cast<uintptr_t>(order) & 3u) != 0)
        return SOL_ERR_ALIGN;
    if (g.NB > 32767 || g.ncand > kMaxCandidates) return SOL_ERR_UNSUPPORTED;
    const size_t need = sol::route_ws_floats(g) * sizeof(float);
    if (workspace == nullptr || ws_bytes < need) return SOL_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SOL_ERR_ALIGN;
    const hipError_t e = sol::launch_route(g, q, k, resolve_scale(scale, g.D), tau, blk_idx, blk_cnt,
                                           totals, order, static_cast<float*>(workspace),
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOL_OK : SOL_ERR_HIP;
}

static sol_status attn_common(const void* q, const void* k, const void* v, const sol_desc* desc,
                              const int16_t* blk_idx, const int32_t* blk_cnt, const int32_t* order,
                              int32_t sink_len, float scale, void* o, float* lse, bool dense,
                              void* stream) {
    sol::Geom g;
    const sol_status st = check_desc(desc, dense ? desc ? desc->N : 0 : sink_len, &g);
    if (st != SOL_OK) return st;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return SOL_ERR_ARG;
    if (!dense && (blk_idx == nullptr || blk_cnt == nullptr)) return SOL_ERR_ARG;
    // O never replaces K or V (other workgroups still read every key row); it
    // may replace Q when the strides match, since each workgroup reads its
    // own query rows before it writes them
    if (o == k || o == v || (o == q && !same_io_strides(desc))) return SOL_ERR_ARG;
    if (std::isnan(scale) || scale < 0.0f || std::isinf(scale)) return SOL_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return SOL_ERR_ALIGN;
    if (!dense && ((reinterpret_cast<uintptr_t>(blk_cnt) & 3u) != 0 ||
                   (reinterpret_cast<uintptr_t>(blk_idx) & 1u) != 0 ||
                   (reinterpret_cast<uintptr_t>(order) & 3u) != 0))
        return SOL_ERR_ALIGN;
    if (!dense && (g.NB > 32767 || g.ncand > kMaxCandidates)) return SOL_ERR_UNSUPPORTED;
    const hipError_t e = sol::launch_attn(g, q, k, v, blk_idx, blk_cnt, dense ? nullptr : order,
                                          resolve_scale(scale, g.D), o, lse, dense,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOL_OK : SOL_ERR_HIP;
}

sol_status sol_attn_fwd(const void* q, const void* k, const void* v, const sol_desc* desc,
                        const int16_t* blk_idx, const int32_t* blk_cnt, const int32_t* order,
                        int32_t sink_len, float scale, void* o, float* lse, void* stream) {
    return attn_common(q, k, v, desc, blk_idx, blk_cnt, order, sink_len, scale, o, lse, false,
                       stream);
}

sol_status sol_attn_dense_fwd(const void* q, const void* k, const void* v, const sol_desc* desc,
                              float scale, void* o, float* lse, void* stream) {
    return attn_common(q, k, v, desc, nullptr, nullptr, nullptr, 0, scale, o, lse, true, stream);
}

sol_status sol_gate_fwd(const void* q, const void* k, const void* v, const sol_desc* desc,
                        const int16_t* blk_idx, const int32_t* blk_cnt, const int32_t* order,
                        int32_t sink_len, float scale, void* o_sparse, void* o_dense,
                        double* stats, void* stream) {
    if (stats == nullptr || o_dense == nullptr) return SOL_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(stats) & 7u) != 0 || !aligned16(o_dense)) return SOL_ERR_ALIGN;
    // both passes read Q, K and V after the other has written its output
    if (o_dense == o_sparse || o_sparse == q || o_sparse == k || o_sparse == v || o_dense == q ||
        o_dense == k || o_dense == v)
        return SOL_ERR_ARG;
    sol_status st = attn_common(q, k, v, desc, blk_idx, blk_cnt, order, sink_len, scale, o_sparse,
                                nullptr, false, stream);
    if (st != SOL_OK) return st;
    st = attn_common(q, k, v, desc, nullptr, nullptr, nullptr, 0, scale, o_dense, nullptr, true,
                     stream);
    if (st != SOL_OK) return st;
    sol::Geom g;
    check_desc(desc, sink_len, &g);
    const hipError_t e = sol::launch_gate(g, o_sparse, o_dense, stats,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOL_OK : SOL_ERR_HIP;
}

sol_status sol_qk_norm_rope_pool(const void* q, const void* k, const sol_desc* desc,
                                 const float* gamma_q, const float* gamma_k, float eps,
                                 const float* rope_cos, const float* rope_sin, int32_t sink_len,
                                 void* q_out, void* k_out, void* workspace, size_t ws_bytes,
                                 void* stream) {
    sol::Geom g;
    const sol_status st = check_desc(desc, sink_len, &g);
    if (st != SOL_OK) return st;
    if (q == nullptr || k == nullptr || q_out == nullptr || k_out == nullptr ||
        gamma_q == nullptr || gamma_k == nullptr || q_out == k_out || q_out == k || k_out == q)
        return SOL_ERR_ARG;
    if ((rope_cos == nullptr) != (rope_sin == nullptr)) return SOL_ERR_ARG;
    if (!(eps >= 0.0f) || std::isinf(eps)) return SOL_ERR_ARG;
    // in place only with identical input and output strides
    if ((q_out == q || k_out == k) && !same_io_strides(desc)) return SOL_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(q_out) || !aligned16(k_out) ||
        !aligned16(gamma_q) || !aligned16(gamma_k) || !aligned16(rope_cos) || !aligned16(rope_sin))
        return SOL_ERR_ALIGN;
    const size_t need = sol::route_ws_floats(g) * sizeof(float);
    if (workspace == nullptr || ws_bytes < need) return SOL_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SOL_ERR_ALIGN;
    const hipError_t e = sol::launch_qk_norm_rope_pool(g, q, k, gamma_q, gamma_k, eps, rope_cos,
                                                       rope_sin, q_out, k_out,
                                                       static_cast<float*>(workspace),
                                                       static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOL_OK : SOL_ERR_HIP;
}

sol_status sol_route_pooled(const sol_desc* desc, float tau, int32_t sink_len, float scale,
                            int16_t* blk_idx, int32_t* blk_cnt, int64_t* totals, int32_t* order,
                            void* workspace, size_t ws_bytes, void* stream) {
    sol::Geom g;
    const sol_status st = check_desc(desc, sink_len, &g);
    if (st != SOL_OK) return st;
    if (blk_idx == nullptr || blk_cnt == nullptr || totals == nullptr) return SOL_ERR_ARG;
    if (std::isnan(tau) || tau < 0.0f || std::isnan(scale) || scale < 0.0f || std::isinf(scale))
        return SOL_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(totals) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(blk_cnt) & 3u) != 0 ||
        (reinterpret_cast<uintptr_t>(blk_idx) & 1u) != 0 ||
        (reinterpret_cast<uintptr_t>(order) & 3u) != 0)
        return SOL_ERR_ALIGN;
    if (g.NB > 32767 || g.ncand > kMaxCandidates) return SOL_ERR_UNSUPPORTED;
    const size_t need = sol::route_ws_floats(g) * sizeof(float);
    if (workspace == nullptr || ws_bytes < need) return SOL_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SOL_ERR_ALIGN;
    const hipError_t e = sol::launch_route_pooled(g, resolve_scale(scale, g.D), tau, blk_idx, blk_cnt,
                                                  totals, order,
                                                  static_cast<float*>(workspace),
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOL_OK : SOL_ERR_HIP;
}

}  // extern "C"

namespace {

// Static routing scratch of sol_route_noalloc (one copy per GPU, held until
// the process ends).  In host code `scratch` names a host-side stand-in, not
// a device address: only the per-device address looked up below is ever
// passed to a kernel.
static __device__ __align__(256) unsigned char scratch[SOL_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, looked up once per device
// with that device current; null on failure.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

sol_status sol_route_noalloc(const void* q, const void* k, const sol_desc* desc, float tau,
                             int32_t sink_len, float scale, int16_t* blk_idx, int32_t* blk_cnt,
                             int64_t* totals, int32_t* order, void* stream) {
    sol::Geom g;
    const sol_status st = check_desc(desc, sink_len, &g);
    if (st != SOL_OK) return st;
    if (q == nullptr || k == nullptr || blk_idx == nullptr || blk_cnt == nullptr || totals == nullptr)
        return SOL_ERR_ARG;
    if (std::isnan(tau) || tau < 0.0f || std::isnan(scale) || scale < 0.0f || std::isinf(scale))
        return SOL_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(totals) & 7u) != 0 ||
        (reinterpret_cast<uintptr_t>(blk_cnt) & 3u) != 0 || (reinterpret_cast<uintptr_t>(blk_idx) & 1u) != 0 ||
        (reinterpret_cast<uintptr_t>(order) & 3u) != 0)
        return SOL_ERR_ALIGN;
    if (g.NB > 32767 || g.ncand > kMaxCandidates) return SOL_ERR_UNSUPPORTED;
    // the same figure as sol_route_workspace_bytes (need plus alignment slack)
    if (sol::route_ws_floats(g) * sizeof(float) + 256 > SOL_NOALLOC_SCRATCH_BYTES) return SOL_ERR_SCRATCH;
    void* ws = device_scratch();
    if (ws == nullptr) return SOL_ERR_HIP;
    const hipError_t e = sol::launch_route(g, q, k, resolve_scale(scale, g.D), tau, blk_idx, blk_cnt,
                                           totals, order, static_cast<float*>(ws),
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOL_OK : SOL_ERR_HIP;
}

const char* sol_status_str(sol_status status) {
    switch (status) {
        case SOL_OK: return "ok";
        case SOL_ERR_ARG: return "invalid argument";
        case SOL_ERR_UNSUPPORTED: return "unsupported shape or size";
        case SOL_ERR_ALIGN: return "misaligned pointer or stride";
        case SOL_ERR_WORKSPACE: return "workspace missing or too small";
        case SOL_ERR_HIP: return "HIP launch failed";
        case SOL_ERR_SCRATCH: return "call needs more scratch than the static buffer holds";
    }
    return "unknown status";
}

}  // extern "C"
