/*
 * Oracle O3: the backward (gradient) of the SDM write/read token loop, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
 * baseline load this file's library. It shares no code, header or constant with the
 * HIP path.
 *
 * The pages make sdm_write_read differentiable in the slot weights, v, beta, the
 * log-decays and the bank (SDMWriteRead, memory_ops.py, diffend page 21; its backward
 * is named, not listed). What the backward computes is therefore fixed by the forward:
 * the gradient of the per-token loop of the SDMWriteRead class docstring (the loop O1
 * runs). This file takes that loop's statements in reverse order and applies the chain
 * rule to each, for a scalar objective
 *     J = sum(grad_out * readings) + sum(grad_bank_final * final bank).
 * Per token, forward (only live tokens; padding touches nothing):
 *     old_w = bank[s_w];  dec_w = exp(g_w) old_w;  ret = sum_w k_w dec_w;
 *     delta = beta (v - ret);  bank[s_w] = dec_w + k_w delta;  out = sum_r q_r bank[s_r].
 * Reverse, with gb the gradient of J with respect to the bank state after the token:
 *     grad_q_r = <grad_out, bank[s_r]>;  gb[s_r] += q_r grad_out     (reading)
 *     gdelta = sum_w k_w gb[s_w];  grad_k_w = <gb[s_w], delta>       (write)
 *     grad_beta = <gdelta, v - ret>;  grad_v = beta gdelta;  gret = -beta gdelta
 *     grad_k_w += <gret, dec_w>;  gdec_w = gb[s_w] + k_w gret          (retrieval)
 *     grad_g_w = <gdec_w, dec_w>;  gb[s_w] = exp(g_w) gdec_w           (decay)
 *     bank[s_w] = old_w                                                (state before it)
 * With one log-decay per token (G = 1), grad_g is the sum over the token's writes.
 * The forward pass saves old_w for every write entry, so the reverse pass restores the
 * bank exactly rather than undoing the decay by division.
 *
 * Layout as in token_loop.c ([P, T, J] stream-major, [P, M, hd] banks), all double:
 *   bank0            the bank before the forward (read only)
 *   grad_out         [P, T, hd] gradient of the readings
 *   grad_bank_final  [P, M, hd] gradient of the final bank, or NULL (zeros)
 *   outputs: grad_bank0 [P, M, hd], grad_k [P, T, W], grad_v [P, T, hd], grad_beta
 *   [P, T], grad_g [P, T, G], grad_q [P, T, R]; every element written (padding tokens 0).
 * Streams [p0, p1). Returns 0, or -1 a slot out of range, -2 a write slot repeated within a
 * token, -3 a bad argument, -4 out of memory.
 *
 * Snapshot storage (sdm_oracle_token_loop_backward_snap, snap_bf16 = 1): the pages let
 * sdm_write_read keep its backward snapshot as bfloat16 rows, rounded to nearest even, on a
 * float32 bank (argument snapshot_quant "bf16", memory_ops.py, page 21), and restore the bank
 * to the dequantized snapshot. Here the snapshot is the saved rows old_w: with snap_bf16 each
 * is stored rounded to bfloat16 (sdm_oracle_round_bf16), and the reverse pass recomputes the
 * token's decayed rows from the rounded rows and restores the bank to them. The forward
 * replay itself runs on the exact rows.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

double sdm_oracle_round_bf16(double x);   /* token_loop.c */

static int backward(int64_t p0, int64_t p1, int64_t T, int64_t W, int64_t R,
                    int64_t G, int64_t hd, int64_t M, const int32_t *k_idx,
                    const double *k_val, const double *v, const double *beta,
                    const double *g, const int32_t *q_idx, const double *q_val,
                    const int32_t *valid, const double *bank0,
                    const double *grad_out, const double *grad_bank_final,
                    double *grad_bank0, double *grad_k, double *grad_v,
                    double *grad_beta, double *grad_g, double *grad_q, int snap_bf16)
{
    if (p0 < 0 || p1 < p0 || T < 0 || W < 1 || R < 1 || hd < 1 || M < 1 || (G != 1 && G != W))
        return -3;
    double *B = (double *)malloc(sizeof(double) * (size_t)(M * hd));
    double *old = (double *)malloc(sizeof(double) * (size_t)((T > 0 ? T : 1) * W * hd));
    double *dec = (double *)malloc(sizeof(double) * (size_t)(W * hd));
    double *ret = (double *)malloc(sizeof(double) * (size_t)hd);
    double *delta = (double *)malloc(sizeof(double) * (size_t)hd);
    double *gdelta = (double *)malloc(sizeof(double) * (size_t)hd);
    double *gret = (double *)malloc(sizeof(double) * (size_t)hd);
    int rc = 0;
    if (!B || !old || !dec || !ret || !delta || !gdelta || !gret) rc = -4;
    for (int64_t p = p0; p < p1 && rc == 0; ++p) {
        const int64_t nvalid = valid ? valid[p] : T;
        double *gb = grad_bank0 + p * M * hd;
        memcpy(B, bank0 + p * M * hd, sizeof(double) * (size_t)(M * hd));
        if (grad_bank_final)
            memcpy(gb, grad_bank_final + p * M * hd, sizeof(double) * (size_t)(M * hd));
        else
            memset(gb, 0, sizeof(double) * (size_t)(M * hd));
        for (int64_t t = 0; t < T; ++t) {   /* padding tokens: zero gradients */
            const int64_t tok = p * T + t;
            memset(grad_k + tok * W, 0, sizeof(double) * (size_t)W);
            memset(grad_q + tok * R, 0, sizeof(double) * (size_t)R);
            memset(grad_g + tok * G, 0, sizeof(double) * (size_t)G);
            memset(grad_v + tok * hd, 0, sizeof(double) * (size_t)hd);
            grad_beta[tok] = 0.0;
        }

        /* forward, saving each written row before its decay */
        for (int64_t t = 0; t < nvalid && rc == 0; ++t) {
            const int64_t tok = p * T + t;
            const int32_t *ks = k_idx + tok * W;
            const double *kv = k_val + tok * W;
            for (int64_t w = 0; w < W && rc == 0; ++w) {
                if (ks[w] < 0 || ks[w] >= M) rc = -1;
                for (int64_t w2 = 0; w2 < w && rc == 0; ++w2)
                    if (ks[w2] == ks[w]) rc = -2;
            }
            for (int64_t r = 0; r < R && rc == 0; ++r)
                if (q_idx[tok * R + r] < 0 || q_idx[tok * R + r] >= M) rc = -1;
            if (rc) break;
            for (int64_t c = 0; c < hd; ++c) ret[c] = 0.0;
            for (int64_t w = 0; w < W; ++w) {
                double *row = B + (int64_t)ks[w] * hd;
                const double gamma = exp(g[tok * G + (G == 1 ? 0 : w)]);
                for (int64_t c = 0; c < hd; ++c)
                    old[(t * W + w) * hd + c] = snap_bf16 ? sdm_oracle_round_bf16(row[c]) : row[c];
                for (int64_t c = 0; c < hd; ++c) {
                    row[c] *= gamma;
                    ret[c] += kv[w] * row[c];
                }
            }
            for (int64_t c = 0; c < hd; ++c) delta[c] = beta[tok] * (v[tok * hd + c] - ret[c]);
            for (int64_t w = 0; w < W; ++w) {
                double *row = B + (int64_t)ks[w] * hd;
                for (int64_t c = 0; c < hd; ++c) row[c] += kv[w] * delta[c];
            }
        }

        /* reverse */
        for (int64_t t = nvalid - 1; t >= 0 && rc == 0; --t) {
            const int64_t tok = p * T + t;
            const int32_t *ks = k_idx + tok * W;
            const double *kv = k_val + tok * W;
            const int32_t *qs = q_idx + tok * R;
            const double *qv = q_val + tok * R;
            const double *go = grad_out + tok * hd;
            const double bt = beta[tok];

            /* reading: out = sum_r q_r bank[s_r], bank after this token's write */
            for (int64_t r = 0; r < R; ++r) {
                const double *row = B + (int64_t)qs[r] * hd;
                double d = 0.0;
                for (int64_t c = 0; c < hd; ++c) d += go[c] * row[c];
                grad_q[tok * R + r] = d;
            }
            for (int64_t r = 0; r < R; ++r) {
                double *grow = gb + (int64_t)qs[r] * hd;
                for (int64_t c = 0; c < hd; ++c) grow[c] += qv[r] * go[c];
            }

            /* recompute the token's decayed rows, retrieval and delta from the saved rows */
            for (int64_t c = 0; c < hd; ++c) ret[c] = 0.0;
            for (int64_t w = 0; w < W; ++w) {
                const double gamma = exp(g[tok * G + (G == 1 ? 0 : w)]);
                for (int64_t c = 0; c < hd; ++c) {
                    dec[w * hd + c] = gamma * old[(t * W + w) * hd + c];
                    ret[c] += kv[w] * dec[w * hd + c];
                }
            }
            for (int64_t c = 0; c < hd; ++c) delta[c] = bt * (v[tok * hd + c] - ret[c]);

            /* write: bank[s_w] = dec_w + k_w delta */
            for (int64_t c = 0; c < hd; ++c) gdelta[c] = 0.0;
            for (int64_t w = 0; w < W; ++w) {
                const double *grow = gb + (int64_t)ks[w] * hd;
                double d = 0.0;
                for (int64_t c = 0; c < hd; ++c) {
                    gdelta[c] += kv[w] * grow[c];
                    d += grow[c] * delta[c];
                }
                grad_k[tok * W + w] = d;
            }
            /* delta = beta (v - ret) */
            double gbeta = 0.0;
            for (int64_t c = 0; c < hd; ++c) {
                gbeta += gdelta[c] * (v[tok * hd + c] - ret[c]);
                grad_v[tok * hd + c] = bt * gdelta[c];
                gret[c] = -bt * gdelta[c];
            }
            grad_beta[tok] = gbeta;
            /* ret = sum_w k_w dec_w; dec_w = exp(g_w) old_w */
            for (int64_t w = 0; w < W; ++w) {
                double *grow = gb + (int64_t)ks[w] * hd;
                double *row = B + (int64_t)ks[w] * hd;
                const double gamma = exp(g[tok * G + (G == 1 ? 0 : w)]);
                double dk = 0.0, dg = 0.0;
                for (int64_t c = 0; c < hd; ++c) {
                    dk += gret[c] * dec[w * hd + c];
                    const double gd = grow[c] + kv[w] * gret[c];
                    dg += gd * dec[w * hd + c];
                    grow[c] = gamma * gd;
                    row[c] = old[(t * W + w) * hd + c];
                }
                grad_k[tok * W + w] += dk;
                grad_g[tok * G + (G == 1 ? 0 : w)] += dg;
            }
        }
    }
    free(B);
    free(old);
    free(dec);
    free(ret);
    free(delta);
    free(gdelta);
    free(gret);
    return rc;
}

int sdm_oracle_token_loop_backward(int64_t p0, int64_t p1, int64_t T, int64_t W, int64_t R,
                                   int64_t G, int64_t hd, int64_t M, const int32_t *k_idx,
                                   const double *k_val, const double *v, const double *beta,
                                   const double *g, const int32_t *q_idx, const double *q_val,
                                   const int32_t *valid, const double *bank0,
                                   const double *grad_out, const double *grad_bank_final,
                                   double *grad_bank0, double *grad_k, double *grad_v,
                                   double *grad_beta, double *grad_g, double *grad_q)
{
    return backward(p0, p1, T, W, R, G, hd, M, k_idx, k_val, v, beta, g, q_idx, q_val, valid, bank0,
                    grad_out, grad_bank_final, grad_bank0, grad_k, grad_v, grad_beta, grad_g, grad_q, 0);
}

int sdm_oracle_token_loop_backward_snap(int64_t p0, int64_t p1, int64_t T, int64_t W, int64_t R,
                                        int64_t G, int64_t hd, int64_t M, const int32_t *k_idx,
                                        const double *k_val, const double *v, const double *beta,
                                        const double *g, const int32_t *q_idx, const double *q_val,
                                        const int32_t *valid, const double *bank0,
                                        const double *grad_out, const double *grad_bank_final,
                                        double *grad_bank0, double *grad_k, double *grad_v,
                                        double *grad_beta, double *grad_g, double *grad_q,
                                        int64_t snap_bf16)
{
    if (snap_bf16 != 0 && snap_bf16 != 1) return -3;
    return backward(p0, p1, T, W, R, G, hd, M, k_idx, k_val, v, beta, g, q_idx, q_val, valid, bank0,
                    grad_out, grad_bank_final, grad_bank0, grad_k, grad_v, grad_beta, grad_g, grad_q,
                    (int)snap_bf16);
}
