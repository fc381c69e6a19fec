/*
 * Reference oracle for masked multi-head attention forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load this
 * library. The product path (the HIP library) never links, loads or calls it, and shares no
 * code, header or table with it.
 *
 * What it computes, for every requested query row (b, hq, i):
 *
 *   O[b,hq,i,:] = sum_{j in J} w_j V[b,kv,j,:],   w_j = exp(s_j - m) / l,
 *   s_j = scale * <Q[b,hq,i,:], K[b,kv,j,:]>,      m = max_{j in J} s_j,
 *   l   = sum_{j in J} exp(s_j - m),               LSE[b,hq,i] = m + ln(l),
 *
 * all in IEEE double precision, where
 *   - kv = hq / (Hq / Hkv) with integer division: grouped-query heads share one key/value
 *     head in consecutive groups, never interleaved ("Triton Cuda Attention", section
 *     "GQA (Grouped-Query Attention)"; multi-query attention is the case Hkv = 1, section "MQA");
 *   - J is the set of visible keys: key j is hidden when causal masking is on and j > i
 *     (the masked multi-head attention CUDA article at wzjinhao.cn/news/73578, section 2.2,
 *     causal mask; "Triton Cuda Attention", section "Causal Attention"), or when a per-batch
 *     valid length is given and j >= valid_len[b] (same article, section 2.2, padding mask);
 *     the two masks combine by intersection (same article, sections 1.3 and 2.2). valid_len
 *     values outside [0, N] are clamped into it.
 *   - The softmax is taken in the three passes the article's naive kernel uses (section 3.1):
 *     first the row maximum, then the sum of exp(s - max), then the weighted sum of V divided
 *     by that sum. The scores are kept from the first pass.
 *   - An explicit mask matrix, when given, is indexed [b, hq, i, j] (the article, section 2.1,
 *     writes the mask as a [B, N, N] matrix broadcast over the scores; section 2.2 lists a
 *     boolean padding mask and, for combined masks, a float matrix added to the score that is
 *     0 where allowed and -inf or a large negative value where not):
 *       keep mask (uint8): key j is visible only where the element is nonzero;
 *       additive mask (double): the element is added to the scaled score s_j, and a key whose
 *       element is -inf is not visible.
 *     It combines with the causal and valid_len masks by intersection.
 *   - A row with no visible key has O = 0 and LSE = -infinity (the article, section 3.2,
 *     recommends a zero output for a fully masked row; the log of an empty sum is -inf).
 *   - LSE is the natural-log log-sum-exp of the scaled scores. The Triton file
 *     tiny_flash_attn_triton.py (kernel _fwd_kernel, the store of L) keeps the same quantity
 *     in base 2 with log2(e) folded into the scores; here it is kept in base e.
 *
 * Inputs are the exact values the device path sees (16-bit inputs widened to double), so no
 * rounding happens here beyond double-precision arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#include <omp.h>

/* The explicit mask row of one query: kind 0 none, 1 keep (uint8), 2 additive (double). */
typedef struct {
    int kind;
    const uint8_t *keep;
    const double *add;
} mask_row;

/* Is key j visible to query i? */
static int key_visible(int64_t i, int64_t j, int causal, int64_t valid, const mask_row *mr)
{
    if (causal && j > i)
        return 0;
    if (j >= valid)
        return 0;
    if (mr->kind == 1 && mr->keep[j] == 0)
        return 0;
    if (mr->kind == 2 && mr->add[j] == -INFINITY)
        return 0;
    return 1;
}

/* One query row, three passes. scores is caller-provided scratch of N doubles. */
static void attend_row(const double *q_row, const double *k_head, const double *v_head,
                       int64_t N, int64_t D, double scale, int causal, int64_t valid, int64_t i,
                       const mask_row *mr, double *scores, double *o_row, double *lse_out)
{
    int64_t j, d, visible = 0;
    double m = -INFINITY, l = 0.0;

    /* pass 1: scores and their maximum */
    for (j = 0; j < N; ++j) {
        if (!key_visible(i, j, causal, valid, mr))
            continue;
        const double *k_row = k_head + j * D;
        double dot = 0.0;
        for (d = 0; d < D; ++d)
            dot += q_row[d] * k_row[d];
        scores[j] = scale * dot;
        if (mr->kind == 2)
            scores[j] += mr->add[j];
        if (scores[j] > m)
            m = scores[j];
        ++visible;
    }
    if (visible == 0) {
        for (d = 0; d < D; ++d)
            o_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    /* pass 2: sum of exponentials relative to the maximum */
    for (j = 0; j < N; ++j) {
        if (!key_visible(i, j, causal, valid, mr))
            continue;
        l += exp(scores[j] - m);
    }
    /* pass 3: normalised weights applied to V */
    for (d = 0; d < D; ++d)
        o_row[d] = 0.0;
    for (j = 0; j < N; ++j) {
        if (!key_visible(i, j, causal, valid, mr))
            continue;
        double w = exp(scores[j] - m) / l;
        const double *v_row = v_head + j * D;
        for (d = 0; d < D; ++d)
            o_row[d] += w * v_row[d];
    }
    *lse_out = m + log(l);
}

/*
 * q: [B,Hq,N,D], k and v: [B,Hkv,N,D], all contiguous doubles on the host.
 * valid_len: int32[B] on the host, or NULL for no padding mask.
 * mask, mask_kind, mask_strides: the explicit mask (kind 0 none, 1 uint8 keep, 2 double
 * additive) with element strides {batch, query head, query row}; element (b, hq, i, j) is at
 * mask + b*s[0] + hq*s[1] + i*s[2] + j. Ignored for kind 0.
 * rows: flat row indices r = (b*Hq + hq)*N + i, or NULL for all B*Hq*N rows in order.
 * out: [nrows, D], lse: [nrows] (row t of the output belongs to rows[t]).
 * threads <= 0 uses the OpenMP default. Returns 0, or -1 on bad arguments.
 */
int oracle_attn_fwd_masked(const double *q, const double *k, const double *v, double *out,
                           double *lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                           double scale, int causal, const int32_t *valid_len, const void *mask,
                           int mask_kind, const int64_t *mask_strides, const int64_t *rows,
                           int64_t nrows, int threads)
{
    if (mask_kind < 0 || mask_kind > 2 || (mask_kind != 0 && (!mask || !mask_strides)))
        return -1;
    if (!q || !k || !v || !out || !lse)
        return -1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || D <= 0 || Hq % Hkv != 0)
        return -1;
    if (rows == NULL)
        nrows = B * Hq * N;
    const int64_t group = Hq / Hkv;
    int bad = 0;
    /* Rows go to threads in chunks of 16 consecutive ones; a short list of rows (a sample of a
     * long sequence) one at a time, so that it still spreads over the threads. */
    const int chunk = nrows >= 1024 ? 16 : 1;

#pragma omp parallel num_threads(threads > 0 ? threads : omp_get_max_threads())
    {
        double *scores = (double *)malloc((size_t)N * sizeof(double));
        if (!scores) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, chunk)
        for (int64_t t = 0; t < nrows; ++t) {
            if (!scores)
                continue;
            int64_t r = rows ? rows[t] : t;
            if (r < 0 || r >= B * Hq * N) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            int64_t i = r % N;
            int64_t bh = r / N;
            int64_t hq = bh % Hq;
            int64_t b = bh / Hq;
            int64_t kv = hq / group;
            int64_t valid = N;
            if (valid_len) {
                valid = valid_len[b];
                if (valid < 0)
                    valid = 0;
                if (valid > N)
                    valid = N;
            }
            mask_row mr = {mask_kind, NULL, NULL};
            if (mask_kind != 0) {
                int64_t off = b * mask_strides[0] + hq * mask_strides[1] + i * mask_strides[2];
                if (mask_kind == 1)
                    mr.keep = (const uint8_t *)mask + off;
                else
                    mr.add = (const double *)mask + off;
            }
            attend_row(q + r * D, k + (b * Hkv + kv) * N * D, v + (b * Hkv + kv) * N * D, N, D,
                       scale, causal, valid, i, &mr, scores, out + t * D, lse + t);
        }
        free(scores);
    }
    return bad ? -1 : 0;
}

/* The same without an explicit mask. */
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *out, double *lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D, double scale,
                    int causal, const int32_t *valid_len, const int64_t *rows, int64_t nrows,
                    int threads)
{
    return oracle_attn_fwd_masked(q, k, v, out, lse, B, Hq, Hkv, N, D, scale, causal, valid_len,
                                  NULL, 0, NULL, rows, nrows, threads);
}

int oracle_max_threads(void)
{
    return omp_get_max_threads();
}


/*
 * Backward pass (test infrastructure only, like everything in this file): the exact gradients
 * of the forward output O with respect to Q, K and V for an upstream gradient dO, i.e. of the
 * scalar sum_{b,hq,i,d} O[b,hq,i,d] * dO[b,hq,i,d]. The pages give the forward only;
 * tiny_flash_attn_triton.py keeps the log-sum-exp for its backward pass. The derivative of the
 * definition above, with w_ij the softmax weights of row i over its visible keys J_i:
 *
 *   dV[b,kv,j]  = sum_{hq in group(kv)} sum_{i : j in J_i} w_ij dO[b,hq,i]
 *   dP_ij       = <dO[b,hq,i], V[b,kv,j]>
 *   D_i         = sum_{j in J_i} w_ij dP_ij
 *   dS_ij       = w_ij (dP_ij - D_i)                 (derivative through the softmax)
 *   dQ[b,hq,i]  = scale * sum_{j in J_i} dS_ij K[b,kv,j]
 *   dK[b,kv,j]  = scale * sum_{hq in group(kv)} sum_{i : j in J_i} dS_ij Q[b,hq,i]
 *
 * Rows with no visible key contribute nothing and get dQ = 0. The weights are recomputed here
 * in the three passes of the forward (no value from the device is used). Work is split over
 * (batch, KV head), so that the dK and dV sums of one KV head belong to one thread.
 * q, dout, dq: [B,Hq,N,D]; k, v, dk, dv: [B,Hkv,N,D]; contiguous doubles. Returns 0 or -1.
 *
 * With an explicit mask (as in oracle_attn_fwd_masked: kind 1 keep bytes, kind 2 additive
 * doubles, element strides (batch, query head, query row), keys contiguous) the visible sets
 * J_i and the scores are the masked forward's: an additive value a_ij enters the score as
 * s_ij = scale q.k + a_ij (so w_ij includes it) and is a constant: dS_ij and every gradient keep
 * the forms above, with dQ and dK carrying only the scale of the q.k term.
 */
int oracle_attn_bwd_masked(const double *q, const double *k, const double *v,
                           const double *dout, double *dq, double *dk, double *dv, int64_t B,
                           int64_t Hq, int64_t Hkv, int64_t N, int64_t D, double scale,
                           int causal, const int32_t *valid_len, const void *mask, int mask_kind,
                           const int64_t *mask_strides, int threads)
{
    if (mask_kind < 0 || mask_kind > 2 || (mask_kind != 0 && (!mask || !mask_strides)))
        return -1;
    if (!q || !k || !v || !dout || !dq || !dk || !dv)
        return -1;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0 || D <= 0 || Hq % Hkv != 0)
        return -1;
    const int64_t group = Hq / Hkv;
    int bad = 0;

#pragma omp parallel num_threads(threads > 0 ? threads : omp_get_max_threads())
    {
        double *w = (double *)malloc((size_t)N * sizeof(double));
        double *dp = (double *)malloc((size_t)N * sizeof(double));
        if (!w || !dp) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t bk = 0; bk < B * Hkv; ++bk) {
            if (!w || !dp)
                continue;
            const int64_t b = bk / Hkv, kv = bk % Hkv;
            const double *k_head = k + bk * N * D, *v_head = v + bk * N * D;
            double *dk_head = dk + bk * N * D, *dv_head = dv + bk * N * D;
            int64_t valid = N;
            if (valid_len) {
                valid = valid_len[b];
                if (valid < 0)
                    valid = 0;
                if (valid > N)
                    valid = N;
            }
            for (int64_t x = 0; x < N * D; ++x)
                dk_head[x] = dv_head[x] = 0.0;
            for (int64_t hq = kv * group; hq < (kv + 1) * group; ++hq) {
                const int64_t bh = b * Hq + hq;
                for (int64_t i = 0; i < N; ++i) {
                    const double *q_row = q + (bh * N + i) * D;
                    const double *do_row = dout + (bh * N + i) * D;
                    double *dq_row = dq + (bh * N + i) * D;
                    int64_t j, d, visible = 0;
                    double m = -INFINITY, l = 0.0, delta = 0.0;
                    mask_row mr = {mask_kind, NULL, NULL};
                    if (mask_kind != 0) {
                        int64_t off = b * mask_strides[0] + hq * mask_strides[1] +
                                      i * mask_strides[2];
                        if (mask_kind == 1)
                            mr.keep = (const uint8_t *)mask + off;
                        else
                            mr.add = (const double *)mask + off;
                    }
                    const mask_row *mrp = &mr;
                    for (d = 0; d < D; ++d)
                        dq_row[d] = 0.0;
                    /* weights, as in the forward's three passes */
                    for (j = 0; j < N; ++j) {
                        if (!key_visible(i, j, causal, valid, mrp))
                            continue;
                        double dot = 0.0;
                        for (d = 0; d < D; ++d)
                            dot += q_row[d] * k_head[j * D + d];
                        w[j] = scale * dot;
                        if (mask_kind == 2)
                            w[j] += mr.add[j];
                        if (w[j] > m)
                            m = w[j];
                        ++visible;
                    }
                    if (visible == 0)
                        continue;
                    for (j = 0; j < N; ++j)
                        if (key_visible(i, j, causal, valid, mrp))
                            l += exp(w[j] - m);
                    for (j = 0; j < N; ++j) {
                        if (!key_visible(i, j, causal, valid, mrp))
                            continue;
                        w[j] = exp(w[j] - m) / l;
                        double dot = 0.0;
                        for (d = 0; d < D; ++d)
                            dot += do_row[d] * v_head[j * D + d];
                        dp[j] = dot;
                        delta += w[j] * dot;
                    }
                    for (j = 0; j < N; ++j) {
                        if (!key_visible(i, j, causal, valid, mrp))
                            continue;
                        const double ds = w[j] * (dp[j] - delta);
                        for (d = 0; d < D; ++d) {
                            dq_row[d] += scale * ds * k_head[j * D + d];
                            dk_head[j * D + d] += scale * ds * q_row[d];
                            dv_head[j * D + d] += w[j] * do_row[d];
                        }
                    }
                }
            }
        }
        free(w);
        free(dp);
    }
    return bad ? -1 : 0;
}

int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dout,
                    double *dq, double *dk, double *dv, int64_t B, int64_t Hq, int64_t Hkv,
                    int64_t N, int64_t D, double scale, int causal, const int32_t *valid_len,
                    int threads)
{
    return oracle_attn_bwd_masked(q, k, v, dout, dq, dk, dv, B, Hq, Hkv, N, D, scale, causal,
                                  valid_len, NULL, 0, NULL, threads);
}
