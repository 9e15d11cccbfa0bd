/*
 * sol.h -- C ABI of the MI355X (gfx950) Sol-Attn block-sparse attention forward.
 *
 * The forward has three parts, all described on the MiniMax-H3 acceleration
 * pages (no page gives code or an API; the operations below are read from
 * their prose):
 *
 *   routing   online, per head, from compressed queries and keys: every
 *             64-token query block picks the key blocks it attends to, with
 *             threshold tau and the diagonal block always kept (clawpit.io
 *             article on the single-4090 run, paragraph on the Sol-Attn
 *             settings; nvlabs.github.io Sol-Engine H3-DataCenter page,
 *             policy paragraph "same online routing"; ty-yang3015 "MiniAcc"
 *             post, "What is Sol attention?": a set of pairs per head).
 *   sink      an exact dense prefix: every query attends to the first S keys
 *             (nvlabs page, policy paragraph: exact 951-token multimodal
 *             prefix sink).
 *   attention softmax attention over the sink keys and the routed keys only,
 *             the two parts merged exactly by log-sum-exp.
 *
 * Tokens form contiguous 64-token blocks in sequence order (nvlabs page: no
 * token reordering).  N is a runtime argument and any N works with the one
 * ahead-of-time build: padding to the 64-aligned length is logical only,
 * padded keys carry exactly zero weight and padded rows are never read or
 * written (tokenfactory.fast post, "The benchmark was not the product": a
 * kernel keyed on the live token count paid a 12-14 s compile per prompt
 * length; the fix was the 64-aligned length with padding masked to zero).
 *
 * Notation:  Blk = 64, NB = ceil(N / 64), scale = 1/sqrt(D) unless given.
 *   j0   = S / 64 (integer division) when S < N, else NB: first key block
 *          holding a non-sink key.  Candidates are the key blocks j0..NB-1.
 *   R(j) = keys [max(64 j, S), min(64 j + 64, N)): the routable keys of block j.
 *   Routing score of query block i and candidate j, float32 in a fixed order:
 *          qbar_i = mean of rows [64 i, min(64 i + 64, N)) of Q   (rows added
 *                   in ascending order from +0, then one correctly rounded divide)
 *          kbar_j = mean of the rows R(j) of K                     (same order)
 *          s_ij   = (fma chain over d = 0..D-1 ascending of qbar_i[d]*kbar_j[d],
 *                   starting from +0) * scale
 *   Selection:  T_i = float32(max_j s_ij - tau);  keep j iff s_ij >= T_i or
 *          j == i.  The pages name tau and a "diagonal threshold" but print no
 *          formula; this gap-to-the-maximum rule is the reading taken.
 *
 * Conventions for every entry point:
 *   - Tensors are device pointers owned by the caller; the library never
 *     allocates or frees memory and keeps no per-call state.  (The one
 *     exception to the second part is sol_route_noalloc, whose scratch is a
 *     static device array per GPU; see there.)
 *   - Q, K, V are [B, N, H, D] bf16 with element strides (sb, sn, sh) shared
 *     by the three tensors (they may be views of one merged QKV projection)
 *     and unit stride along D; O has its own strides.  Rows >= N are never
 *     read (loads past them return zero) and never written.
 *   - Packed variable-length batches (mixed prompt lengths in one call;
 *     tokenfactory.fast post, "The benchmark was not the product": served
 *     traffic mixes prompt lengths, and one build must serve them all): when
 *     desc->cu_seqlens is not NULL, the B samples lie back to back in
 *     [T, H, D] tensors, T = desc->total_rows.  Sample b is rows
 *     cu_seqlens[b] .. cu_seqlens[b + 1] - 1, its length n_b between 0 and N
 *     (N is then the longest sample), and every rule above applies to each
 *     sample on its own with N = n_b: its own blocks, sink, candidates and
 *     routing, and no attention across samples.  qkv_sb and o_sb must be 0.
 *     Per-block and per-row outputs keep the fixed-length layout, sized by
 *     the longest sample: blk_idx [B, H, NB, NB], blk_cnt and order
 *     [B, H, NB], lse [B, H, N] with NB = ceil(N / 64).  Past a sample's own
 *     blocks blk_cnt is 0 and order holds the block's own index; lse rows
 *     >= n_b and O rows outside every sample are never written.
 *     cu_seqlens is device int32 [B + 1], non-decreasing, cu_seqlens[B] <=
 *     T, total_rows < 2^31.  The kernels clamp each sample to [0, T) and to
 *     at most N rows, so offsets that break these rules cannot make an
 *     access leave the buffers (the results of such samples are then
 *     unspecified).  A NULL cu_seqlens gives the fixed-length batch above
 *     and total_rows is ignored.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise the host.
 *   - Errors come back as a status code; nothing is printed.  Argument checks
 *     run on the host before any HIP call, so a rejected call touches no
 *     device state.  SOL_ERR_HIP means a kernel launch failed.
 *   - D must be 64 or 128.  Base pointers and strides must give 16-byte
 *     aligned rows.
 *   - Thread safety: calls on different streams may run concurrently.  The
 *     only mutable global state is sol_route_noalloc's static scratch array
 *     on each GPU and the cache of its per-device address (filled under a
 *     mutex): overlapping sol_route_noalloc calls on one GPU race on that
 *     array; every other entry point works only on the caller's buffers.
 */
#ifndef SOL_H
#define SOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SOL_BLOCK 64

typedef enum {
    SOL_OK = 0,
    SOL_ERR_ARG = 1,          /* null pointer, non-positive size, negative S, NaN or negative tau,
                                 nonzero batch stride or negative T with cu_seqlens               */
    SOL_ERR_UNSUPPORTED = 2,  /* D not 64/128, stride along D != 1, a size beyond the limits    */
    SOL_ERR_ALIGN = 3,        /* a pointer or stride that breaks 16-byte row alignment          */
    SOL_ERR_WORKSPACE = 4,    /* workspace null or smaller than sol_route_workspace_bytes()     */
    SOL_ERR_HIP = 5,          /* a kernel launch reported an error                              */
    SOL_ERR_SCRATCH = 6       /* sol_route_noalloc: the call needs more scratch than the
                                 library's static buffer holds (SOL_NOALLOC_SCRATCH_BYTES)     */
} sol_status;

typedef struct {
    int32_t B, N, H, D;               /* batch, true sequence length, heads, head width    */
    int64_t qkv_sb, qkv_sn, qkv_sh;   /* element strides of Q, K and V (unit along D)      */
    int64_t o_sb, o_sn, o_sh;         /* element strides of O (unit along D)               */
    const int32_t* cu_seqlens;        /* packed variable-length batch: device int32 [B+1]
                                         row offsets of the samples, or NULL (fixed N)     */
    int64_t total_rows;               /* T, rows of the packed tensors (with cu_seqlens)   */
} sol_desc;

/* Number of 64-token blocks, ceil(N / 64) (0 for N <= 0). */
int32_t sol_num_blocks(int32_t N);

/* Device workspace that sol_route needs, in bytes: room for the pooled
 * queries and keys, 2 * B * H * NB * D float32 (sol_qk_norm_rope_pool writes
 * both there; sol_route itself stores only the key means, its scoring pass
 * pools the queries on chip), then scratch for the partial totals of the
 * scoring pass (16 bytes per 12 query blocks per (batch, head)), plus
 * alignment.  0 for an invalid desc. */
size_t sol_route_workspace_bytes(const sol_desc* desc);

/*
 * sol_route -- online block routing (pooling, pooled scores, selection).
 *
 *   q, k      [B, N, H, D] bf16 device tensors (strides in desc).
 *   tau       threshold >= 0 in scaled-logit units; +INFINITY keeps every
 *             candidate (routing disabled).  NaN or negative: SOL_ERR_ARG.
 *   sink_len  S >= 0; S = 0 disables the sink, S >= N makes every key a sink
 *             key (no candidates, every list empty).
 *   scale     softmax scale of the scores; 0 means 1/sqrt(D).
 *   blk_idx   out, device int16 [B, H, NB, NB]: row (b, h, i) holds the
 *             selected key blocks of query block i in ascending order in its
 *             first blk_cnt[b, h, i] entries; the rest of the row is not
 *             written.  Requires NB <= 32767.
 *   blk_cnt   out, device int32 [B, H, NB].
 *   totals    out, device int64 [2]: totals[0] = sum of blk_cnt (routed block
 *             pairs); totals[1] = attended (query, key) pairs over valid rows,
 *             sink included.  Exact integers, so densities are exact.
 *   order     out, optional (NULL to skip), device int32 [B, H, NB]: the
 *             attention schedule.  Row (b, h) is a permutation of the query
 *             blocks 0..NB-1 with non-increasing blk_cnt (longest list first;
 *             blocks of equal length in no fixed order).  It changes only the
 *             timing of sol_attn_fwd, never its results.
 *   workspace device scratch of at least sol_route_workspace_bytes(desc)
 *             bytes, 256-byte aligned; contents on entry are ignored.
 *
 * Limits: NB - j0 <= 4096 candidates (N up to about 262k tokens).
 */
sol_status sol_route(const void* q, const void* k, const sol_desc* desc, float tau,
                     int32_t sink_len, float scale, int16_t* blk_idx, int32_t* blk_cnt,
                     int64_t* totals, int32_t* order, void* workspace, size_t ws_bytes,
                     void* stream);

/*
 * sol_attn_fwd -- sink + routed block-sparse attention forward.
 *
 *   q, k, v   [B, N, H, D] bf16 device tensors (strides in desc).
 *   blk_idx,  the lists written by sol_route for the same B, N, H and
 *   blk_cnt   sink_len (entries must be ascending candidates in [j0, NB)).
 *   order     optional (NULL: sequence order) schedule written by sol_route;
 *             each row must be a permutation of 0..NB-1 (for a packed
 *             sample: its first ceil(n_b / 64) entries a permutation of its
 *             own blocks, as sol_route writes them).  Query blocks of one
 *             (batch, head) are processed in this order; results do not
 *             depend on it.
 *   sink_len  S >= 0 as for sol_route.
 *   scale     softmax scale; 0 means 1/sqrt(D).
 *   o         out, [B, N, H, D] bf16 (strides in desc): for each valid query
 *             row, softmax attention over keys [0, min(S, N)) and the keys
 *             R(j) of every listed block j, rounded to bf16 (nearest even).
 *             o may be q itself when the O strides equal the Q/K/V strides
 *             (each query block reads its own rows before it writes them);
 *             o == k, o == v, or o == q with other strides: SOL_ERR_ARG.
 *             Other overlaps of o with an input are not detected and give
 *             unspecified results.
 *   lse       out, optional (NULL to skip), float32 [B, H, N]: natural-log
 *             log-sum-exp of the scaled logits over the same keys.
 */
sol_status sol_attn_fwd(const void* q, const void* k, const void* v, const sol_desc* desc,
                        const int16_t* blk_idx, const int32_t* blk_cnt, const int32_t* order,
                        int32_t sink_len, float scale, void* o, float* lse, void* stream);

/*
 * sol_attn_dense_fwd -- full softmax attention (routing disabled), the path
 * the pages keep for the first denoising steps and first layers (nvlabs page,
 * policy paragraph).  Arguments as for sol_attn_fwd; every key is attended.
 */
sol_status sol_attn_dense_fwd(const void* q, const void* k, const void* v, const sol_desc* desc,
                              float scale, void* o, float* lse, void* stream);

/*
 * sol_gate_fwd -- the sparse-vs-dense correctness gate: one sparse forward
 * (as sol_attn_fwd) into o_sparse and one dense forward (as
 * sol_attn_dense_fwd) into o_dense of the same inputs, then their error
 * statistics over the valid rows (tokenfactory.fast post, "Verification
 * that catches what the metrics miss": the gate compares the two outputs
 * inside one attention call; clawpit.io article, paragraph on the Sol-Attn
 * settings: reported as maximum, mean and relative L2 error).
 *
 *   o_sparse, o_dense  out, [B, N, H, D] bf16 with the O strides of desc;
 *                      distinct buffers, neither of them q, k or v (the
 *                      second pass reads the inputs after the first has
 *                      written): SOL_ERR_ARG otherwise.
 *   stats     out, device float64 [7], 8-byte aligned: [0] max |s - d|,
 *             [1] sum |s - d|, [2] sum (s - d)^2, [3] sum d^2, [4] number
 *             of elements compared, [5] mean |s - d| = [1] / [4], [6]
 *             relative L2 error sqrt([2] / [3]) (0 when a divisor is 0).
 *             The maximum is exact; the sums are float64 atomics whose last
 *             bits depend on completion order.
 * Other arguments and errors as for sol_attn_fwd.
 */
sol_status sol_gate_fwd(const void* q, const void* k, const void* v, const sol_desc* desc,
                        const int16_t* blk_idx, const int32_t* blk_cnt, const int32_t* order,
                        int32_t sink_len, float scale, void* o_sparse, void* o_dense,
                        double* stats, void* stream);

/*
 * sol_qk_norm_rope_pool -- the producer right before the path: QK-norm and
 * RoPE of the query and key rows, written as the bf16 Q and K that routing
 * and attention read, and in the same pass the block means that routing
 * scores (tokenfactory.fast post, "Custom kernels": a fused QK-norm plus
 * RoPE kernel; clawpit.io article, paragraph on the Sol-Attn settings:
 * routing from compressed queries and keys).  With it, routing never reads
 * Q and K again: sol_route_pooled starts from the means.  The pages define
 * neither operation; the plainest reading is taken and fixed in float32:
 *
 *   For every valid row x (one head, D channels) at position t of its
 *   sample, with weights gamma (gamma_q for Q, gamma_k for K):
 *     ss   = running float32 sum over d = 0 .. D-1 ascending of x_d * x_d,
 *            from +0 (each square is exact; one rounding per step)
 *     r    = 1 / sqrt(fma(ss, 1/D, eps))   (each step correctly rounded)
 *     y_d  = (x_d * r) * gamma_d            (per-head RMS normalisation)
 *     RoPE on the channel pairs (2i, 2i+1), with c = cos[t][i], s = sin[t][i]:
 *       o_2i   = fma(y_2i, c, -(y_2i+1 * s))
 *       o_2i+1 = fma(y_2i, s,   y_2i+1 * c)
 *     out  = o rounded to bf16 (nearest even)
 *   Block means, float32, of the rounded outputs: exactly the pooling of
 *   sol_route applied to q_out and k_out (rows added in ascending order from
 *   +0, one divide; key means over R(j) only), written into workspace.
 *
 *   q, k         in, [B, N, H, D] bf16 (Q/K/V strides of desc), or packed.
 *   q_out, k_out out, bf16 with the O strides of desc; may equal q and k
 *                (in place) when the O strides equal the Q/K/V strides.
 *   gamma_q/_k   device float32 [D], 16-byte aligned.
 *   eps          >= 0, finite.
 *   rope_cos/sin device float32 [N, D/2] (row t = position t of a sample),
 *                16-byte aligned; both NULL: no RoPE (o = y).
 *   sink_len     S, for the key means over R(j).
 *   workspace    as for sol_route (sol_route_workspace_bytes(desc) bytes,
 *                256-byte aligned): receives the block means.
 */
sol_status sol_qk_norm_rope_pool(const void* q, const void* k, const sol_desc* desc,
                                 const float* gamma_q, const float* gamma_k, float eps,
                                 const float* rope_cos, const float* rope_sin, int32_t sink_len,
                                 void* q_out, void* k_out, void* workspace, size_t ws_bytes,
                                 void* stream);

/*
 * sol_route_pooled -- sol_route from block means already in the workspace
 * (written by sol_qk_norm_rope_pool for the same desc and sink_len): scores,
 * selection, lists, totals and schedule exactly as sol_route computes them
 * on q_out and k_out, without reading Q or K.  The means are only read; the
 * workspace's scratch tail is written.  Arguments and errors as for
 * sol_route.
 */
sol_status sol_route_pooled(const sol_desc* desc, float tau, int32_t sink_len, float scale,
                            int16_t* blk_idx, int32_t* blk_cnt, int64_t* totals, int32_t* order,
                            void* workspace, size_t ws_bytes, void* stream);

/*
 * sol_route_noalloc -- sol_route without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, and harnesses that forbid allocation.  The pooled means and
 * partial totals that sol_route keeps in the caller's workspace live instead
 * in a static device array of SOL_NOALLOC_SCRATCH_BYTES bytes that the
 * library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine.
 *
 * Results are identical, bit for bit, to sol_route with a workspace.  A call
 * whose sol_route_workspace_bytes(desc) exceeds SOL_NOALLOC_SCRATCH_BYTES
 * returns SOL_ERR_SCRATCH before any launch (the pages' shape
 * [1, 38247, 56, 128] needs 34.3 MB).  The scratch of the current device is
 * used, so `stream` must belong to the current device.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (on different
 * streams or from different threads) race and give unspecified results;
 * calls ordered on one stream are safe.  No part of the array needs to start
 * at zero (every call writes what it reads).  The first call on a device
 * looks up the array's address on that device (hipGetSymbolAddress); a
 * failure there returns SOL_ERR_HIP.  Other arguments and errors as for
 * sol_route.
 */
#define SOL_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)

sol_status sol_route_noalloc(const void* q, const void* k, const sol_desc* desc, float tau,
                             int32_t sink_len, float scale, int16_t* blk_idx, int32_t* blk_cnt,
                             int64_t* totals, int32_t* order, void* stream);

/* Static, human-readable name of a status code. */
const char* sol_status_str(sol_status status);

#ifdef __cplusplus
}
#endif

#endif /* SOL_H */
