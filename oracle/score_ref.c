/*
 * CPU oracle, float32 definitions: pooled block scores, and the QK-norm + RoPE
 * producer (second half of this file).  TEST INFRASTRUCTURE ONLY: nothing on
 * the product path links or calls this file.
 *
 * Online routing in Sol-Attn compares compressed (block-pooled) queries with
 * compressed keys, per head (clawpit.io article on the single-4090 run,
 * paragraph on the Sol-Attn settings; ty-yang3015 blog, "What is Sol
 * attention?").  The pages give no formula; the score of query block i against
 * key block j is read here as the dot product of the two block means, times
 * the softmax scale, computed in float32 in one fixed order:
 *
 *     acc = +0
 *     for d = 0 .. D-1 (ascending):  acc = fmaf(qbar[i][d], kbar[j][d], acc)
 *     score = acc * scale            (one float32 rounding)
 *
 * fmaf is the C99 fused multiply-add: one correct rounding per step.  Built
 * with -ffp-contract=off so the final multiply stays a plain float32 multiply.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

void oracle_block_scores(const float *qbar, const float *kbar, int64_t nq, int64_t nk,
                         int64_t d, float scale, float *out)
{
    for (int64_t i = 0; i < nq; ++i) {
        const float *qi = qbar + i * d;
        for (int64_t j = 0; j < nk; ++j) {
            const float *kj = kbar + j * d;
            float acc = 0.0f;
            for (int64_t t = 0; t < d; ++t)
                acc = fmaf(qi[t], kj[t], acc);
            out[i * nk + j] = acc * scale;
        }
    }
}

/*
 * QK-norm + RoPE in float32.  QK-norm plus RoPE is the fused op the
 * tokenfactory.fast post ("Custom kernels") names right before attention; the
 * pages define neither, so the reading is per-head RMS normalisation with a
 * weight per channel, then the rotation of channel pairs (2i, 2i + 1) by the
 * angle whose cosine and sine the caller tables give for the row's position.
 * One row x of D bf16 values, each step one float32 rounding, in this order:
 *
 *   ss    = +0;  for d = 0 .. D-1 ascending:  ss = fmaf(x[d], x[d], ss)
 *           (the plain running sum of squares: a bf16 square is exact in
 *           float32, so the fused and the unfused step round alike)
 *   r     = 1 / sqrtf(fmaf(ss, 1/D, eps))
 *   y[d]  = (x[d] * r) * gamma[d]
 *   o[2i] = fmaf(y[2i], c, -(y[2i+1] * s)),  o[2i+1] = fmaf(y[2i], s, y[2i+1] * c)
 *   out   = o rounded to bf16, nearest even
 *
 * x and out are rows x d bf16 bit patterns; cosv / sinv are rows x d/2 (the
 * row's position already applied) or both NULL for no rotation.
 */
static float bf16_to_f32(uint16_t b)
{
    const uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

void oracle_qk_norm_rope(const uint16_t *x, int64_t rows, int64_t d, const float *gamma,
                         float eps, const float *cosv, const float *sinv, uint16_t *out)
{
    for (int64_t t = 0; t < rows; ++t) {
        const uint16_t *xr = x + t * d;
        float ss = 0.0f;
        for (int64_t e = 0; e < d; ++e) {
            const float v = bf16_to_f32(xr[e]);
            ss = fmaf(v, v, ss);
        }
        const float r = 1.0f / sqrtf(fmaf(ss, 1.0f / (float)d, eps));
        float y[512];
        for (int64_t e = 0; e < d; ++e)
            y[e] = (bf16_to_f32(xr[e]) * r) * gamma[e];
        if (cosv != NULL) {
            for (int64_t i = 0; i < d / 2; ++i) {
                const float c = cosv[t * (d / 2) + i], s = sinv[t * (d / 2) + i];
                const float a = y[2 * i], b = y[2 * i + 1];
                y[2 * i] = fmaf(a, c, -(b * s));
                y[2 * i + 1] = fmaf(a, s, b * c);
            }
        }
        for (int64_t e = 0; e < d; ++e)
            out[t * d + e] = f32_to_bf16_rne(y[e]);
    }
}
