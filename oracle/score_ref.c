/*
 * CPU oracle, pooled block scores.  TEST INFRASTRUCTURE ONLY: nothing on the
 * product path links or calls this file.
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
