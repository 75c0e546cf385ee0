/*
 * Oracle O1: the SDM write/read forward as a token-by-token recurrence, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
 * baseline load this file's library. It shares no code, header or constant with the
 * HIP path.
 *
 * Definition followed: the per-token loop in the SDMWriteRead class docstring of
 * memory_ops.py (sparse-delta-memory 2.0.0 wheel, diffend page 21). For each token,
 * each written bank row is first multiplied by the exponential of its log-decay
 * (only written rows decay); the retrieved vector is the k-weighted sum of those
 * decayed rows; the write error is beta times (v minus retrieved); each written row
 * then becomes its decayed value plus its weight times that error; the reading is
 * the q-weighted sum of the read rows after the write. The chunked form on the
 * pages reproduces this loop up to floating-point rounding.
 *
 * Layout (all row-major, one stream after another):
 *   k_idx  int32  [P, T, W]   write slots, stream-local rows in [0, M)
 *   k_val  double [P, T, W]
 *   v      double [P, T, hd]
 *   beta   double [P, T]
 *   g      double [P, T, G]   G = 1 (one log-decay per token) or W (one per write)
 *   q_idx  int32  [P, T, R]
 *   q_val  double [P, T, R]
 *   valid  int32  [P] or NULL (NULL: every token valid). Tokens t >= valid[p] are
 *          padding: they touch no row and their reading is 0 (the module docstring
 *          of memory_ops.py: padding is inert and outputs zeros).
 *   bank   double [P, M, hd]  advanced in place to its final state
 *   out    double [P, T, hd]  readings
 *
 * Streams [p0, p1) are processed; each stream owns its bank [M, hd] (the per-stream
 * slot ranges of sdm_write_read's num_memory_slots argument).
 *
 * Returns 0, or a negative code on a violated caller contract: -1 a slot id out of
 * range, -2 a write slot repeated within one token (the op requires distinct write
 * slots per token), -3 a bad argument, -4 out of memory.
 *
 * O1b, the same loop under the bf16 storage contract (sdm_oracle_token_loop_bf16): the
 * pages keep a bfloat16 bank in bfloat16 and round each written bank row once per chunk,
 * at its decay-and-write store, and return the readings in the bank dtype (phase2_kernels
 * .py docstring and _sdm_dual_matmul, diffend page 23; sdm_write_read's docstring, page
 * 21). O1b therefore runs the exact fp64 token loop and, at the end of every chunk of
 * `chunk` tokens (and at the last token), rounds every row written in that chunk to the
 * nearest bfloat16 (ties to even); each reading is rounded to bfloat16. It isolates the
 * error that bfloat16 storage itself causes from arithmetic error.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Nearest bfloat16 (8 significant bits, ties to even) of a finite double, exactly
 * (one rounding: no intermediate float). */
double sdm_oracle_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);                 /* x = m 2^e, 0.5 <= |m| < 1 */
    double s = ldexp(m, 8);                  /* 128 <= |s| < 256: the 8 kept bits */
    double r = nearbyint(s);                 /* default rounding mode: ties to even */
    return ldexp(r, e - 8);
}

/* bank_stride: elements from stream p's bank to stream p + 1's (M * hd for one bank per
 * stream; 0 for one bank shared by every stream, whose slot sets the caller keeps
 * disjoint). */
static int token_loop(int64_t p0, int64_t p1, int64_t T, int64_t W, int64_t R, int64_t G,
                      int64_t hd, int64_t M, int64_t bank_stride, const int32_t *k_idx,
                      const double *k_val, const double *v, const double *beta, const double *g,
                      const int32_t *q_idx, const double *q_val, const int32_t *valid,
                      double *bank, double *out, int64_t round_chunk)
{
    if (p0 < 0 || p1 < p0 || T < 0 || W < 1 || R < 1 || hd < 1 || M < 1 || (G != 1 && G != W))
        return -3;
    double *retrieved = (double *)malloc(sizeof(double) * (size_t)hd);
    double *delta = (double *)malloc(sizeof(double) * (size_t)hd);
    char *touched = round_chunk > 0 ? (char *)calloc((size_t)M, 1) : NULL;
    if (!retrieved || !delta || (round_chunk > 0 && !touched)) {
        free(retrieved);
        free(delta);
        free(touched);
        return -4;
    }
    int rc = 0;
    for (int64_t p = p0; p < p1 && rc == 0; ++p) {
        double *B = bank + p * bank_stride;
        int64_t nvalid = valid ? valid[p] : T;
        for (int64_t t = 0; t < T && rc == 0; ++t) {
            int64_t tok = p * T + t;
            double *o = out + tok * hd;
            if (t >= nvalid) {
                for (int64_t c = 0; c < hd; ++c) o[c] = 0.0;
                continue;
            }
            const int32_t *ks = k_idx + tok * W;
            const double *kv = k_val + tok * W;
            const int32_t *qs = q_idx + tok * R;
            const double *qv = q_val + tok * R;
            for (int64_t w = 0; w < W; ++w) {
                if (ks[w] < 0 || ks[w] >= M) { rc = -1; break; }
                for (int64_t w2 = 0; w2 < w; ++w2)
                    if (ks[w2] == ks[w]) { rc = -2; break; }
            }
            for (int64_t r = 0; r < R && rc == 0; ++r)
                if (qs[r] < 0 || qs[r] >= M) rc = -1;
            if (rc) break;

            /* decay the written rows: bank[k] = exp(g) * bank[k] (the "read" rows) */
            for (int64_t w = 0; w < W; ++w) {
                double gamma = exp(g[tok * G + (G == 1 ? 0 : w)]);
                double *row = B + (int64_t)ks[w] * hd;
                for (int64_t c = 0; c < hd; ++c) row[c] *= gamma;
                if (touched) touched[ks[w]] = 1;
            }
            /* retrieved = sum_w k_w * read_w */
            for (int64_t c = 0; c < hd; ++c) retrieved[c] = 0.0;
            for (int64_t w = 0; w < W; ++w) {
                const double *row = B + (int64_t)ks[w] * hd;
                for (int64_t c = 0; c < hd; ++c) retrieved[c] += kv[w] * row[c];
            }
            /* delta_v = beta * (v - retrieved) */
            for (int64_t c = 0; c < hd; ++c) delta[c] = beta[tok] * (v[tok * hd + c] - retrieved[c]);
            /* bank[k] = read + k (x) delta_v */
            for (int64_t w = 0; w < W; ++w) {
                double *row = B + (int64_t)ks[w] * hd;
                for (int64_t c = 0; c < hd; ++c) row[c] += kv[w] * delta[c];
            }
            /* reading = sum_r q_r * bank[q_r], after the write */
            for (int64_t c = 0; c < hd; ++c) o[c] = 0.0;
            for (int64_t r = 0; r < R; ++r) {
                const double *row = B + (int64_t)qs[r] * hd;
                for (int64_t c = 0; c < hd; ++c) o[c] += qv[r] * row[c];
            }
            if (touched) {
                for (int64_t c = 0; c < hd; ++c) o[c] = sdm_oracle_round_bf16(o[c]);
                if ((t + 1) % round_chunk == 0 || t + 1 == nvalid) {
                    for (int64_t s = 0; s < M; ++s) {
                        if (!touched[s]) continue;
                        double *row = B + s * hd;
                        for (int64_t c = 0; c < hd; ++c) row[c] = sdm_oracle_round_bf16(row[c]);
                        touched[s] = 0;
                    }
                }
            }
        }
    }
    free(retrieved);
    free(delta);
    free(touched);
    return rc;
}

int sdm_oracle_token_loop(int64_t p0, int64_t p1, int64_t T, int64_t W, int64_t R, int64_t G,
                          int64_t hd, int64_t M, const int32_t *k_idx, const double *k_val,
                          const double *v, const double *beta, const double *g,
                          const int32_t *q_idx, const double *q_val, const int32_t *valid,
                          double *bank, double *out)
{
    return token_loop(p0, p1, T, W, R, G, hd, M, M * hd, k_idx, k_val, v, beta, g, q_idx, q_val,
                      valid, bank, out, 0);
}

int sdm_oracle_token_loop_bf16(int64_t p0, int64_t p1, int64_t T, int64_t W, int64_t R, int64_t G,
                               int64_t hd, int64_t M, int64_t chunk, const int32_t *k_idx,
                               const double *k_val, const double *v, const double *beta,
                               const double *g, const int32_t *q_idx, const double *q_val,
                               const int32_t *valid, double *bank, double *out)
{
    if (chunk < 1) return -3;
    return token_loop(p0, p1, T, W, R, G, hd, M, M * hd, k_idx, k_val, v, beta, g, q_idx, q_val,
                      valid, bank, out, chunk);
}

/* Either loop over one [M, hd] bank shared by every stream (chunk 0: O1, else O1b). */
int sdm_oracle_token_loop_shared(int64_t p0, int64_t p1, int64_t T, int64_t W, int64_t R,
                                 int64_t G, int64_t hd, int64_t M, int64_t chunk,
                                 const int32_t *k_idx, const double *k_val, const double *v,
                                 const double *beta, const double *g, const int32_t *q_idx,
                                 const double *q_val, const int32_t *valid, double *bank,
                                 double *out)
{
    if (chunk < 0) return -3;
    return token_loop(p0, p1, T, W, R, G, hd, M, 0, k_idx, k_val, v, beta, g, q_idx, q_val,
                      valid, bank, out, chunk);
}
