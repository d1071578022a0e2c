/*
 * eta_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow and deliberately unoptimised fp64 reference of the Elastic
 * Threshold Attention (ETA) decode step, written from the pages that describe
 * arXiv:2609.20888 ("Elastic Threshold Attention: Learned Contextual Sparsity
 * for Long-Context Decoding"):
 *   - the evolve.pub review, "Methodology Assessment": Eq. 1 (linear threshold
 *     predictor on the concatenated post-RoPE queries), Eq. 2 (sigmoid gate
 *     sigma(beta*(S - tau))) and Eq. 3 (multiplicative gating S * m);
 *   - the same review, Q&A "What is ETA?": at inference, a whole KV block is
 *     skipped when the best score any of its keys could reach is below tau;
 *   - the same review, "Summary": the screen uses cached per-block centroid,
 *     variance and max-norm metadata;
 *   - the paper abstract (montaan.com paper page, "Abstract"): constant-time
 *     block screening from cached bounds with a geometric and a probabilistic
 *     part, logits under the threshold multiplied down to zero, frozen per-head
 *     thresholds after offline calibration.
 * Where the pages leave a step open, the reading taken is stated at the
 * function. Only the test suite, the smoke check and the benchmark's CPU
 * baseline may load this file's library; the GPU path never does.
 *
 * Every loop runs in the order the definition reads; no blocking, fusion or
 * reordering. Build: gcc -O2 -ffp-contract=off -shared -fPIC.
 */
#include "eta_oracle.h"

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bfloat16 is the upper half of an IEEE binary32: widen by a 16-bit shift. */
double eta_oracle_bf16_to_f64(uint16_t bits) {
    uint32_t w = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Element (t, i) of a [T_cap][d] key or value slab, widened to fp64. */
static double kv_at(const void *X, int kv_dtype, int d, long t, int i) {
    if (kv_dtype == ORACLE_KV_BF16) {
        const uint16_t *p = (const uint16_t *)X;
        return eta_oracle_bf16_to_f64(p[t * (long)d + i]);
    }
    const float *p = (const float *)X;
    return (double)p[t * (long)d + i];
}

/* Eq. 1 of the review's "Methodology Assessment": tau = qbar W + b, where
 * qbar concatenates the post-RoPE queries of all H heads of one batch row and
 * W maps that H*d vector to one threshold per head. With no predictor (the
 * abstract's calibrated deployment) tau is the frozen per-head constant. */
void eta_oracle_predict_tau(int B, int H, int d, const float *q, const float *W,
                            const float *bias, double *tau) {
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            double acc = (double)bias[h];
            if (W != NULL) {
                for (int g = 0; g < H; ++g) {
                    for (int i = 0; i < d; ++i) {
                        long row = (long)g * d + i; /* position in qbar */
                        double qv = (double)q[((long)b * H + g) * d + i];
                        double wv = (double)W[row * H + h];
                        acc += qv * wv;
                    }
                }
            }
            tau[(long)b * H + h] = acc;
        }
    }
}

/* Cached block metadata (review "Summary": centroid / variance / max-norm).
 * Reading: block beta holds tokens [beta*bs, min(T, (beta+1)*bs)); the
 * centroid is the mean key; the variance is ONE scalar per block, the mean
 * over the block's tokens and the d dimensions of (k - centroid)^2
 * (population form, second pass after the mean); max-norm is the largest key
 * L2 norm. A partial last block uses only its present tokens. */
int eta_oracle_block_meta(int T, int d, int bs, int kv_dtype, const void *K,
                          double *centroid, double *var, double *maxnorm) {
    int nblk = (T + bs - 1) / bs;
    for (int blk = 0; blk < nblk; ++blk) {
        long t0 = (long)blk * bs;
        long t1 = t0 + bs;
        if (t1 > T) t1 = T;
        double n = (double)(t1 - t0);
        double *c = centroid + (long)blk * d;

        for (int i = 0; i < d; ++i) c[i] = 0.0;
        for (long t = t0; t < t1; ++t)
            for (int i = 0; i < d; ++i) c[i] += kv_at(K, kv_dtype, d, t, i);
        for (int i = 0; i < d; ++i) c[i] /= n;

        double sq = 0.0;
        double best = 0.0;
        for (long t = t0; t < t1; ++t) {
            double norm2 = 0.0;
            for (int i = 0; i < d; ++i) {
                double k = kv_at(K, kv_dtype, d, t, i);
                double dev = k - c[i];
                sq += dev * dev;
                norm2 += k * k;
            }
            double norm = sqrt(norm2);
            if (norm > best) best = norm;
        }
        var[blk] = sq / (n * (double)d);
        maxnorm[blk] = best;
    }
    return nblk;
}

/* Block score bound (abstract: the screen uses cached bounds that are partly
 * geometric, partly probabilistic; Q&A "What is ETA?": the highest score any key
 * of the block could reach). With s = 1/sqrt(d):
 *   geometric     U_geo  = s * |q| * maxnorm          (Cauchy-Schwarz: no key
 *                                                     of the block can score
 *                                                     higher)
 *   probabilistic U_prob = s * (q.c + z * |q| * sqrt(var))  (centroid score
 *                                                     plus z in-block standard
 *                                                     deviations, isotropic)
 * COMBINED uses min(U_geo, U_prob); GEO uses U_geo alone. */
void eta_oracle_bounds(int nblk, int d, const float *q_unit, const double *centroid,
                       const double *var, const double *maxnorm, double z, int mode,
                       double *U) {
    double s = 1.0 / sqrt((double)d);
    double qn2 = 0.0;
    for (int i = 0; i < d; ++i) qn2 += (double)q_unit[i] * (double)q_unit[i];
    double qn = sqrt(qn2);
    for (int blk = 0; blk < nblk; ++blk) {
        double u_geo = s * qn * maxnorm[blk];
        if (mode == ORACLE_BOUND_GEO) {
            U[blk] = u_geo;
            continue;
        }
        double qc = 0.0;
        for (int i = 0; i < d; ++i) qc += (double)q_unit[i] * centroid[(long)blk * d + i];
        double u_prob = s * (qc + z * qn * sqrt(var[blk]));
        U[blk] = (u_prob < u_geo) ? u_prob : u_geo;
    }
}

/* Centroid-relative geometric bound (abstract: cached geometric bounds; review
 * "Summary": centroid and max-norm metadata), the reading of "max-norm" as the
 * largest distance of a block's keys from its centroid.
 * Per block: the centroid c is the mean key (first pass), then
 *   maxdev = max over the block's tokens of |k - c|      (second pass).
 * Same block ranges as eta_oracle_block_meta. */
int eta_oracle_block_maxdev(int T, int d, int bs, int kv_dtype, const void *K, double *maxdev) {
    int nblk = (T + bs - 1) / bs;
    double *c = (double *)malloc(sizeof(double) * (size_t)d);
    for (int blk = 0; blk < nblk; ++blk) {
        long t0 = (long)blk * bs;
        long t1 = t0 + bs;
        if (t1 > T) t1 = T;
        double n = (double)(t1 - t0);
        for (int i = 0; i < d; ++i) c[i] = 0.0;
        for (long t = t0; t < t1; ++t)
            for (int i = 0; i < d; ++i) c[i] += kv_at(K, kv_dtype, d, t, i);
        for (int i = 0; i < d; ++i) c[i] /= n;
        double best = 0.0;
        for (long t = t0; t < t1; ++t) {
            double dist2 = 0.0;
            for (int i = 0; i < d; ++i) {
                double dev = kv_at(K, kv_dtype, d, t, i) - c[i];
                dist2 += dev * dev;
            }
            double dist = sqrt(dist2);
            if (dist > best) best = dist;
        }
        maxdev[blk] = best;
    }
    free(c);
    return nblk;
}

/* The centered bound: every key k of the block has q.k = q.c + q.(k - c) <=
 * q.c + |q| * |k - c| (Cauchy-Schwarz), so
 *   U_cen = s * (q.c + |q| * maxdev)
 * is never below the block's best score; it is taken together with the
 * max-norm bound, U = min(U_geo, U_cen), and like U_geo alone it can miss no
 * block whose best key reaches tau. */
void eta_oracle_bounds_centered(int nblk, int d, const float *q_unit, const double *centroid,
                                const double *maxnorm, const double *maxdev, double *U) {
    double s = 1.0 / sqrt((double)d);
    double qn2 = 0.0;
    for (int i = 0; i < d; ++i) qn2 += (double)q_unit[i] * (double)q_unit[i];
    double qn = sqrt(qn2);
    for (int blk = 0; blk < nblk; ++blk) {
        double u_geo = s * qn * maxnorm[blk];
        double qc = 0.0;
        for (int i = 0; i < d; ++i) qc += (double)q_unit[i] * centroid[(long)blk * d + i];
        double u_cen = s * (qc + qn * maxdev[blk]);
        U[blk] = (u_cen < u_geo) ? u_cen : u_geo;
    }
}

/* Hard skip (Q&A "What is ETA?"): a block whose bound is below tau is not
 * loaded at all. Reading: admit iff U >= tau (a tie is kept); NaN admits
 * nothing. The list is ascending. */
int eta_oracle_screen(int nblk, const double *U, double tau, int32_t *idx) {
    int cnt = 0;
    for (int blk = 0; blk < nblk; ++blk) {
        if (U[blk] >= tau) idx[cnt++] = blk;
    }
    return cnt;
}

/* Grouped heads (a reading: the pages measure the fraction of blocks fetched
 * when the selections of several heads are fetched together). A
 * block is loaded for a KV head when any of its query heads admits it; each
 * query head then attends over that union with its own gate, so blocks that
 * only another head admitted enter through the gate's floor. */
int eta_oracle_union(int g, const int32_t *lists, const int32_t *cnts, int stride, int nblk,
                     int32_t *out) {
    int cnt = 0;
    for (int blk = 0; blk < nblk; ++blk) {
        int hit = 0;
        for (int j = 0; j < g && !hit; ++j)
            for (int a = 0; a < cnts[j] && !hit; ++a)
                if (lists[(long)j * stride + a] == blk) hit = 1;
        if (hit) out[cnt++] = blk;
    }
    return cnt;
}

/* Eq. 2 of the review's "Methodology Assessment": m = sigma(beta*(S - tau)),
 * the logistic function. The hard form (beta -> infinity) is the step
 * S >= tau. */
double eta_oracle_gate(double S, double tau, double beta, int hard) {
    if (hard) return (S >= tau) ? 1.0 : 0.0;
    double x = beta * (S - tau);
    return 1.0 / (1.0 + exp(-x));
}

/* Decode attention over the admitted blocks (abstract; Q&A "What is ETA?").
 * For every token j < T of every admitted block, in ascending order:
 *   S_j  = s * q.k_j                     (s = 1/sqrt(d))
 *   S'_j = S_j * gate(S_j)               (Eq. 3: multiplicative suppression;
 *                                         a suppressed logit tends to 0, i.e.
 *                                         weight e^0 = 1, not to -inf)
 * then ordinary softmax attention on S':
 *   mu = max_j S'_j,  l = sum_j exp(S'_j - mu),
 *   out = sum_j exp(S'_j - mu) v_j / l,  lse = mu + log(l).
 * Reading for an empty admitted set: out = 0 and lse = -inf. */
void eta_oracle_attend(int T, int d, int bs, int kv_dtype, const float *q_unit,
                       const void *K, const void *V, double tau, const int32_t *idx,
                       int cnt, double gate_beta, int gate_hard, double *out,
                       double *lse) {
    double s = 1.0 / sqrt((double)d);
    for (int i = 0; i < d; ++i) out[i] = 0.0;
    if (cnt <= 0) {
        *lse = -INFINITY;
        return;
    }

    /* pass 1: the largest gated logit */
    double mu = -INFINITY;
    for (int a = 0; a < cnt; ++a) {
        long t0 = (long)idx[a] * bs;
        long t1 = t0 + bs;
        if (t1 > T) t1 = T;
        for (long t = t0; t < t1; ++t) {
            double dot = 0.0;
            for (int i = 0; i < d; ++i) dot += (double)q_unit[i] * kv_at(K, kv_dtype, d, t, i);
            double S = s * dot;
            double Sg = S * eta_oracle_gate(S, tau, gate_beta, gate_hard);
            if (Sg > mu) mu = Sg;
        }
    }

    /* pass 2: softmax weights and the weighted sum of values */
    double l = 0.0;
    for (int a = 0; a < cnt; ++a) {
        long t0 = (long)idx[a] * bs;
        long t1 = t0 + bs;
        if (t1 > T) t1 = T;
        for (long t = t0; t < t1; ++t) {
            double dot = 0.0;
            for (int i = 0; i < d; ++i) dot += (double)q_unit[i] * kv_at(K, kv_dtype, d, t, i);
            double S = s * dot;
            double Sg = S * eta_oracle_gate(S, tau, gate_beta, gate_hard);
            double p = exp(Sg - mu);
            l += p;
            for (int i = 0; i < d; ++i) out[i] += p * kv_at(V, kv_dtype, d, t, i);
        }
    }
    for (int i = 0; i < d; ++i) out[i] /= l;
    *lse = mu + log(l);
}

/* Training-time forward (review "Methodology Assessment", Eq. 1-3 applied to
 * every query token; abstract: in training a logit under the threshold is
 * multiplied down to zero): the T_q queries are the last T_q positions of the T_k
 * keys, and query t (position T_k - T_q + t) sees keys 0 .. its position.
 * For each query: out and lse are the gated attention of eta_oracle_attend
 * over its visible keys (all their blocks admitted), and gate_sum is the sum
 * of the gates eta_oracle_gate(S_j) over those keys.
 * Q float32 [T_q][d]; tau fp64 [T_q]; out fp64 [T_q][d]; lse, gate_sum
 * fp64 [T_q]. Returns 0, or -1 when scratch memory cannot be had. */
int eta_oracle_prefill(int T_q, int T_k, int d, int kv_dtype, const float *Q, const void *K,
                       const void *V, const double *tau, double gate_beta, int gate_hard,
                       double *out, double *lse, double *gate_sum) {
    const int bs = 64;
    double s = 1.0 / sqrt((double)d);
    int nblk_max = (T_k + bs - 1) / bs;
    int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nblk_max > 0 ? nblk_max : 1));
    if (idx == NULL) return -1;
    for (int b = 0; b < nblk_max; ++b) idx[b] = b;
    for (int t = 0; t < T_q; ++t) {
        int n = T_k - T_q + t + 1; /* visible keys */
        const float *q = Q + (long)t * d;
        eta_oracle_attend(n, d, bs, kv_dtype, q, K, V, tau[t], idx, (n + bs - 1) / bs,
                          gate_beta, gate_hard, out + (long)t * d, lse + t);
        double gs = 0.0;
        for (long j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int i = 0; i < d; ++i) dot += (double)q[i] * kv_at(K, kv_dtype, d, j, i);
            gs += eta_oracle_gate(s * dot, tau[t], gate_beta, gate_hard);
        }
        gate_sum[t] = gs;
    }
    free(idx);
    return 0;
}
