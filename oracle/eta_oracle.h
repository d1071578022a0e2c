/*
 * eta_oracle.h -- TEST INFRASTRUCTURE, not part of the product.
 *
 * Plain, slow, fp64 CPU reference of the Elastic Threshold Attention (ETA)
 * block-sparse decode step (arXiv:2609.20888). Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load this library. It shares
 * no code, header, table or constant with the GPU library; the only thing the
 * two sides share is the seeded input data they are both handed.
 *
 * Every function works on ONE (batch, head) unit unless stated otherwise, and
 * every array is row-major and contiguous:
 *   q_unit   float32 [d]           post-RoPE query of the unit
 *   K, V     [T_cap][d]            keys / values of the unit, float32 or the
 *                                  raw 16-bit patterns of bfloat16 (kv_dtype)
 *   centroid double  [nblk][d]     per-block metadata (fp64, token-major)
 *   var, maxnorm double [nblk]
 * Nothing here allocates memory that outlives a call, and nothing is global.
 */
#ifndef ETA_ORACLE_H
#define ETA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_KV_F32 = 0, ORACLE_KV_BF16 = 1 };
enum { ORACLE_BOUND_COMBINED = 0, ORACLE_BOUND_GEO = 1 };

/* Exact widening of one bfloat16 bit pattern to fp64. */
double eta_oracle_bf16_to_f64(uint16_t bits);

/* Eq. 1: tau[b][h] = bias[h] + sum_{g<H, i<d} q[b][g][i] * W[g*d+i][h].
 * q float32 [B][H][d], W float32 [H*d][H] (NULL = static per-head tau),
 * bias float32 [H], tau fp64 [B][H]. */
void eta_oracle_predict_tau(int B, int H, int d, const float *q, const float *W,
                            const float *bias, double *tau);

/* Per-block metadata of one unit over its first T tokens (blocks of bs):
 * centroid = mean key, var = mean over tokens and dims of (k - centroid)^2
 * (population, two-pass), maxnorm = largest key L2 norm. Returns nblk. */
int eta_oracle_block_meta(int T, int d, int bs, int kv_dtype, const void *K,
                          double *centroid, double *var, double *maxnorm);

/* Upper bound U of the scaled score s*q.k (s = 1/sqrt(d)) of every key in
 * each block: geometric (Cauchy-Schwarz) s*|q|*maxnorm, probabilistic
 * s*(q.centroid + z*|q|*sqrt(var)); COMBINED takes the smaller of the two,
 * GEO only the first. */
void eta_oracle_bounds(int nblk, int d, const float *q_unit, const double *centroid,
                       const double *var, const double *maxnorm, double z, int mode,
                       double *U);

/* Largest distance of a block's keys from the block's centroid, per block (two
 * passes: centroid, then max |k - centroid|). Returns nblk. */
int eta_oracle_block_maxdev(int T, int d, int bs, int kv_dtype, const void *K, double *maxdev);

/* Centered bound: min(s*|q|*maxnorm, s*(q.centroid + |q|*maxdev)), both sides
 * guaranteed (Cauchy-Schwarz about the origin and about the centroid). */
void eta_oracle_bounds_centered(int nblk, int d, const float *q_unit, const double *centroid,
                                const double *maxnorm, const double *maxdev, double *U);

/* Admission: block b is admitted iff U[b] >= tau. Writes the admitted block
 * ids in ascending order to idx (room for nblk) and returns their count. */
int eta_oracle_screen(int nblk, const double *U, double tau, int32_t *idx);

/* Union of the admitted lists of the g query heads that share one KV head
 * (grouped-query attention): lists[j][0..cnts[j]) for j < g, each ascending,
 * rows `stride` apart. Writes the ascending union to out (room for nblk) and
 * returns its length. */
int eta_oracle_union(int g, const int32_t *lists, const int32_t *cnts, int stride, int nblk,
                     int32_t *out);

/* Eq. 2 gate at one logit: sigmoid(beta*(S - tau)), or the step S >= tau. */
double eta_oracle_gate(double S, double tau, double beta, int hard);

/* Gated softmax attention over the tokens (< T) of the admitted blocks:
 * S_j = s*q.k_j, S'_j = S_j * gate(S_j), out = softmax(S') . V, lse = log of
 * the softmax denominator. An empty admitted set gives out = 0, lse = -inf. */
void eta_oracle_attend(int T, int d, int bs, int kv_dtype, const float *q_unit,
                       const void *K, const void *V, double tau, const int32_t *idx,
                       int cnt, double gate_beta, int gate_hard, double *out,
                       double *lse);

/* Training-time forward of a whole (row, head): the T_q queries Q [T_q][d]
 * (float32) are the last T_q positions of the T_k keys; query t sees keys
 * 0 .. T_k - T_q + t. Per query: out [d] and lse as eta_oracle_attend over its
 * visible keys, and gate_sum = the sum of gate(S_j) over them. tau fp64
 * [T_q]; out fp64 [T_q][d]; lse, gate_sum fp64 [T_q]. Returns 0, or -1 when
 * scratch memory cannot be had (freed before returning). */
int eta_oracle_prefill(int T_q, int T_k, int d, int kv_dtype, const float *Q, const void *K,
                       const void *V, const double *tau, double gate_beta, int gate_hard,
                       double *out, double *lse, double *gate_sum);

#ifdef __cplusplus
}
#endif
#endif /* ETA_ORACLE_H */
