/*
 * oracle.c -- fp64 CPU oracle for causal scaled dot-product multi-head
 * self-attention (forward and backward) and for the pre-norm attention
 * sublayer around it.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * definition that the HIP kernels are checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or constant with the GPU library, and it
 * includes nothing from it.
 *
 * Everything is double precision, naive loops, in the order the definition
 * is written.  OpenMP only splits independent (batch, head) pairs or
 * independent rows across threads; no loop is blocked, fused or reordered.
 *
 * Sources (the pages this follows):
 *  - "LLM from scratch" CS336 tutorial (lmnt.cn), section 5.1 model.py,
 *    class CausalSelfAttention.forward: scores are q times k-transpose
 *    multiplied by 1/sqrt(head dim); entries where the lower-triangular
 *    ones-matrix is zero are filled with -inf; softmax over the last axis;
 *    the weights multiply v.  Section 3.3 of the same page: -inf on the upper
 *    triangle so that those weights become 0 after the softmax.
 *  - "Train Your Own LLM from Scratch" (fishgap), section 1: the causal mask
 *    is tril(ones(block_size, block_size)), so the diagonal is kept (j <= i).
 *  - Backward: the pages only run loss.backward() through this op (CS336
 *    tutorial, section 5.2 train.py).  The gradient is therefore the exact
 *    derivative of the forward above; the formulas below are the softmax
 *    chain rule, written out, and are pinned by finite differences in the
 *    tests, not by any printed formula.
 *  - Sublayer: CS336 tutorial section 5.1, class LayerNorm (biased variance,
 *    eps added under the square root), class Block.forward (x + attn(ln_1(x))),
 *    CausalSelfAttention (c_attn, chunk into q,k,v, view per head, c_proj).
 *
 * Layout: q, k, v, o, dO, dq, dk, dv are contiguous [B][H][T][D];
 * lse and delta are [B][H][T].  lse is the natural-log log-sum-exp of the
 * scaled scores of each row (a reading: the pages never define it).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void set_threads(int64_t nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads((int)nthreads);
#else
    (void)nthreads;
#endif
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* First key row i sees.  window = 0: every earlier key (the causal mask of
 * CS336 section 5.1).  window = W > 0: the W most recent keys, i - W < j <= i
 * (the sliding-window attention that nanochat section 9 lists; the band of the
 * causal mask, read with the diagonal kept as above). */
static int64_t first_key(int64_t i, int64_t window)
{
    return (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;
}

/* One row of the causal softmax: p[j] for j = j0..i, from scores s[j].
 * Returns m (the row max) and writes Z (the normaliser) so that
 * lse = m + log(Z).  Keys j > i (and j < j0 in a window) are masked (-inf)
 * and carry weight exactly 0, so they are simply not part of the sum. */
static void causal_softmax_row(const double* Qi, const double* K, int64_t i,
                               int64_t j0, int64_t D, double scale, double* s, double* p,
                               double* m_out, double* Z_out)
{
    double m = -INFINITY;
    for (int64_t j = j0; j <= i; ++j) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += Qi[d] * K[j * D + d];
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }
    double Z = 0.0;
    for (int64_t j = j0; j <= i; ++j) Z += exp(s[j] - m);
    for (int64_t j = j0; j <= i; ++j) p[j] = exp(s[j] - m) / Z;
    *m_out = m;
    *Z_out = Z;
}

/* Forward: o = softmax(mask(scale * q k^T)) v, lse = log sum exp of the row. */
void oracle_attn_fwd(const double* q, const double* k, const double* v,
                     double* o, double* lse, int64_t B, int64_t H, int64_t T,
                     int64_t D, double scale, int64_t window, int64_t nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double* Q = q + bh * T * D;
        const double* K = k + bh * T * D;
        const double* V = v + bh * T * D;
        double* O = o + bh * T * D;
        double* L = lse + bh * T;
        double* s = (double*)malloc((size_t)T * sizeof(double));
        double* p = (double*)malloc((size_t)T * sizeof(double));
        for (int64_t i = 0; i < T; ++i) {
            double m, Z;
            const int64_t j0 = first_key(i, window);
            causal_softmax_row(Q + i * D, K, i, j0, D, scale, s, p, &m, &Z);
            for (int64_t d = 0; d < D; ++d) {
                double acc = 0.0;
                for (int64_t j = j0; j <= i; ++j) acc += p[j] * V[j * D + d];
                O[i * D + d] = acc;
            }
            L[i] = m + log(Z);
        }
        free(s);
        free(p);
    }
}

/* Backward of L = sum(dO * O) through the forward above.
 *   dP_ij = dO_i . v_j               (j <= i)
 *   Delta_i = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - Delta_i)   (softmax Jacobian)
 *   dq_i  = scale sum_{j<=i} dS_ij k_j
 *   dk_j  = scale sum_{i>=j} dS_ij q_i
 *   dv_j  =       sum_{i>=j} P_ij dO_i
 * delta receives Delta (row-wise). */
void oracle_attn_bwd(const double* q, const double* k, const double* v,
                     const double* dO, double* dq, double* dk, double* dv,
                     double* delta, int64_t B, int64_t H, int64_t T, int64_t D,
                     double scale, int64_t window, int64_t nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double* Q = q + bh * T * D;
        const double* K = k + bh * T * D;
        const double* V = v + bh * T * D;
        const double* G = dO + bh * T * D;
        double* dQ = dq + bh * T * D;
        double* dK = dk + bh * T * D;
        double* dV = dv + bh * T * D;
        double* Dl = delta + bh * T;
        double* s = (double*)malloc((size_t)T * sizeof(double));
        double* p = (double*)malloc((size_t)T * sizeof(double));
        double* dp = (double*)malloc((size_t)T * sizeof(double));
        memset(dK, 0, (size_t)(T * D) * sizeof(double));
        memset(dV, 0, (size_t)(T * D) * sizeof(double));
        for (int64_t i = 0; i < T; ++i) {
            double m, Z;
            const int64_t j0 = first_key(i, window);
            causal_softmax_row(Q + i * D, K, i, j0, D, scale, s, p, &m, &Z);
            double Delta = 0.0;
            for (int64_t j = j0; j <= i; ++j) {
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d) acc += G[i * D + d] * V[j * D + d];
                dp[j] = acc;
                Delta += p[j] * dp[j];
            }
            Dl[i] = Delta;
            for (int64_t d = 0; d < D; ++d) dQ[i * D + d] = 0.0;
            for (int64_t j = j0; j <= i; ++j) {
                double dS = p[j] * (dp[j] - Delta);
                for (int64_t d = 0; d < D; ++d) {
                    dQ[i * D + d] += scale * dS * K[j * D + d];
                    dK[j * D + d] += scale * dS * Q[i * D + d];
                    dV[j * D + d] += p[j] * G[i * D + d];
                }
            }
        }
        free(s);
        free(p);
        free(dp);
    }
}

/* ------------------------------------------------------------------------ */
/* Attention dropout.  CS336 tutorial, section 5.1: CausalSelfAttention      */
/* applies its nn.Dropout to the softmax weights, att = dropout(att), before  */
/* att @ v (every configuration on the pages sets p = 0).  In training mode   */
/* that is inverted dropout: each weight is kept with probability 1 - p and  */
/* scaled by 1 / (1 - p), else zeroed; the softmax normaliser and lse are     */
/* those of the undropped weights.                                            */
/* The keep decisions must be the same in the forward and the backward, so   */
/* they come from a counter-based generator, Philox4x32-10 (Salmon, Moraes,  */
/* Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011;     */
/* the Random123 definition), read as follows (this scheme is a choice):     */
/*   counter (j / 8, i, b * H + h, 0), key (seed mod 2^32, seed / 2^32);      */
/*   element j % 8 takes 16-bit half (j % 2) of output word (j % 8) / 2;      */
/*   kept iff that value >= p16, where p16 = round(p * 65536) < 65536;        */
/*   kept weights are scaled by 65536 / (65536 - p16).                        */
/* ------------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        const uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        const uint32_t y1 = (uint32_t)p1;
        const uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        const uint32_t y3 = (uint32_t)p0;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
        k0 += 0x9E3779B9u;  /* the key schedule (Weyl sequence) */
        k1 += 0xBB67AE85u;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* 1 if weight (bh, i, j) is kept. */
int oracle_dropout_keep(uint64_t seed, int64_t p16, int64_t bh, int64_t i, int64_t j)
{
    const uint32_t ctr[4] = {(uint32_t)(j / 8), (uint32_t)i, (uint32_t)bh, 0u};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t r[4];
    oracle_philox4x32_10(ctr, key, r);
    const uint32_t u = (r[(j % 8) / 2] >> (16 * (j % 2))) & 0xFFFFu;
    return (int64_t)u >= p16;
}

/* Forward with dropout: o_i = sum_j P_ij keep_ij / (1 - p) v_j; lse as without.
 * bh0: the global (batch, head) index of the first pair given (the draws are
 * indexed by it), so that a slice of a larger batch can be checked alone. */
void oracle_attn_fwd_dropout(const double* q, const double* k, const double* v, double* o,
                             double* lse, int64_t B, int64_t H, int64_t T, int64_t D,
                             double scale, int64_t window, int64_t p16, uint64_t seed,
                             int64_t bh0, int64_t nthreads)
{
    const double keep_scale = 65536.0 / (65536.0 - (double)p16);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double* Qh = q + bh * T * D;
        const double* Kh = k + bh * T * D;
        const double* Vh = v + bh * T * D;
        double* O = o + bh * T * D;
        double* s = (double*)malloc((size_t)T * sizeof(double));
        double* w = (double*)malloc((size_t)T * sizeof(double));
        for (int64_t i = 0; i < T; ++i) {
            double m, Z;
            const int64_t j0 = first_key(i, window);
            causal_softmax_row(Qh + i * D, Kh, i, j0, D, scale, s, w, &m, &Z);
            for (int64_t j = j0; j <= i; ++j)  /* the dropped weights */
                w[j] = oracle_dropout_keep(seed, p16, bh0 + bh, i, j) ? w[j] * keep_scale : 0.0;
            for (int64_t d = 0; d < D; ++d) {
                double sum = 0.0;
                for (int64_t j = j0; j <= i; ++j) sum += w[j] * Vh[j * D + d];
                O[i * D + d] = sum;
            }
            lse[bh * T + i] = m + log(Z);
        }
        free(s);
        free(w);
    }
}

/* Backward with dropout, for the forward above (pd = the dropped weights):
 *   dv_j  = sum_i pd_ij dO_i
 *   dP_ij = keep_ij / (1 - p) * (dO_i . v_j)     (gradient of the undropped P)
 *   Delta_i = sum_j P_ij dP_ij  (= dO_i . o_i)
 *   dS_ij = P_ij (dP_ij - Delta_i);  dq, dk as without dropout. */
void oracle_attn_bwd_dropout(const double* q, const double* k, const double* v,
                             const double* dO, double* dq, double* dk, double* dv, double* delta,
                             int64_t B, int64_t H, int64_t T, int64_t D, double scale,
                             int64_t window, int64_t p16, uint64_t seed, int64_t bh0,
                             int64_t nthreads)
{
    const double keep_scale = 65536.0 / (65536.0 - (double)p16);
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const double* Qh = q + bh * T * D;
        const double* Kh = k + bh * T * D;
        const double* Vh = v + bh * T * D;
        const double* Gh = dO + bh * T * D;
        double* dQh = dq + bh * T * D;
        double* dKh = dk + bh * T * D;
        double* dVh = dv + bh * T * D;
        double* s = (double*)malloc((size_t)T * sizeof(double));
        double* w = (double*)malloc((size_t)T * sizeof(double));
        double* gw = (double*)malloc((size_t)T * sizeof(double));
        double* mk = (double*)malloc((size_t)T * sizeof(double));
        memset(dKh, 0, (size_t)(T * D) * sizeof(double));
        memset(dVh, 0, (size_t)(T * D) * sizeof(double));
        for (int64_t i = 0; i < T; ++i) {
            double m, Z;
            const int64_t j0 = first_key(i, window);
            causal_softmax_row(Qh + i * D, Kh, i, j0, D, scale, s, w, &m, &Z);
            double Dl = 0.0;
            for (int64_t j = j0; j <= i; ++j) {
                mk[j] = oracle_dropout_keep(seed, p16, bh0 + bh, i, j) ? keep_scale : 0.0;
                double sum = 0.0;
                for (int64_t d = 0; d < D; ++d) sum += Gh[i * D + d] * Vh[j * D + d];
                gw[j] = mk[j] * sum;
                Dl += w[j] * gw[j];
            }
            delta[bh * T + i] = Dl;
            for (int64_t d = 0; d < D; ++d) dQh[i * D + d] = 0.0;
            for (int64_t j = j0; j <= i; ++j) {
                const double ds = w[j] * (gw[j] - Dl);
                for (int64_t d = 0; d < D; ++d) {
                    dQh[i * D + d] += scale * ds * Kh[j * D + d];
                    dKh[j * D + d] += scale * ds * Qh[i * D + d];
                    dVh[j * D + d] += w[j] * mk[j] * Gh[i * D + d];
                }
            }
        }
        free(s);
        free(w);
        free(gw);
        free(mk);
    }
}

/* ------------------------------------------------------------------------ */
/* Decode: one new token per sequence against its key/value cache.            */
/* nanochat, section 8 (inference engine): the KV cache is kept in FA3's      */
/* native (B, T, H, D) layout; a prompt is prefilled into it, then tokens are */
/* produced one at a time, each attending to every cached position up to and  */
/* including its own (CS336 tutorial, section 7.4, names the KV cache among   */
/* the inference-side optimisations).  The token of sequence b is at position */
/* len_b - 1 and its key and value are already in the cache, so its output is */
/* row len_b - 1 of the causal forward above over that sequence; with a       */
/* window W > 0, the W most recent positions.                                 */
/* q, o: [B][H][D]; kc, vc: [B][Tmax][H][D]; lens: [B] (0 <= len_b <= Tmax);  */
/* lse: [B][H].  len_b = 0 (nothing cached): o = 0 and lse = -inf.            */
/* ------------------------------------------------------------------------ */
void oracle_attn_decode(const double* q, const double* kc, const double* vc,
                        const int64_t* lens, double* o, double* lse, int64_t B,
                        int64_t H, int64_t Tmax, int64_t D, double scale,
                        int64_t window, int64_t nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        const int64_t len = lens[b];
        const double* Q = q + bh * D;
        double* O = o + bh * D;
        if (len <= 0) {
            for (int64_t d = 0; d < D; ++d) O[d] = 0.0;
            lse[bh] = -INFINITY;
            continue;
        }
        const int64_t last = len - 1;  /* the new token's position */
        const int64_t j0 = first_key(last, window);
        double* s = (double*)malloc((size_t)len * sizeof(double));
        double m = -INFINITY;
        for (int64_t j = j0; j <= last; ++j) {
            const double* Kj = kc + ((b * Tmax + j) * H + h) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += Q[d] * Kj[d];
            s[j] = dot * scale;
            if (s[j] > m) m = s[j];
        }
        double Z = 0.0;
        for (int64_t j = j0; j <= last; ++j) Z += exp(s[j] - m);
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int64_t j = j0; j <= last; ++j)
                acc += exp(s[j] - m) / Z * vc[((b * Tmax + j) * H + h) * D + d];
            O[d] = acc;
        }
        lse[bh] = m + log(Z);
        free(s);
    }
}

/* ------------------------------------------------------------------------ */
/* RoPE and QK-norm on the query and key rows of every head.                 */
/* nanochat, section 9, lists RoPE position encoding and QK norm (with a     */
/* factor of 1.2) among the attention's parts; the pages give no formulas,    */
/* so the standard forms are taken (readings):                                */
/*  - RoPE rotates the pair of columns (i, i + D/2), i < D/2, of the row at   */
/*    position p = pos0 + t by the angle p * base^(-2i/D):                    */
/*        y_i       = x_i cos - x_{i+D/2} sin                                 */
/*        y_{i+D/2} = x_i sin + x_{i+D/2} cos                                 */
/*  - QK norm divides the row by its root mean square, sqrt(mean(x^2) + eps), */
/*    with no learned weight, and multiplies by `gain` (1.2 for queries in    */
/*    the pages' wording, 1 for keys).                                        */
/* Rotation keeps the root mean square, so the two commute.                   */
/* x, y, dy, dx: [B][H][T][D]; use_rope / use_norm switch each part.          */
/* ------------------------------------------------------------------------ */
static void rope_angle(int64_t p, int64_t i, int64_t D, double base, double* c, double* s)
{
    const double theta = (double)p * pow(base, -2.0 * (double)i / (double)D);
    *c = cos(theta);
    *s = sin(theta);
}

void oracle_rope_qknorm_fwd(const double* x, double* y, int64_t B, int64_t H, int64_t T,
                            int64_t D, int64_t pos0, double base, int64_t use_rope,
                            int64_t use_norm, double gain, double eps)
{
    const int64_t half = D / 2;
    for (int64_t row = 0; row < B * H * T; ++row) {
        const int64_t t = row % T;
        const double* X = x + row * D;
        double* Y = y + row * D;
        double r = 1.0;
        if (use_norm) {
            double ss = 0.0;
            for (int64_t d = 0; d < D; ++d) ss += X[d] * X[d];
            r = gain / sqrt(ss / (double)D + eps);
        }
        for (int64_t i = 0; i < half; ++i) {
            double c = 1.0, s = 0.0;
            if (use_rope) rope_angle(pos0 + t, i, D, base, &c, &s);
            Y[i] = r * (X[i] * c - X[i + half] * s);
            Y[i + half] = r * (X[i] * s + X[i + half] * c);
        }
    }
}

/* Gradient of sum(dy * y) with respect to x for the map above.  With
 * z = R x (rotation) and y = gain * z / rms(x), rms(x) = sqrt(mean(x^2) + eps):
 *   dz = (gain / rms) dy - z * (gain / rms^3) * mean(dy * z)   (norm)
 *   dx = R^T dz                                                (rotation)
 * (rotation keeps the norm, so mean(x^2) = mean(z^2)). */
void oracle_rope_qknorm_bwd(const double* x, const double* dy, double* dx, int64_t B,
                            int64_t H, int64_t T, int64_t D, int64_t pos0, double base,
                            int64_t use_rope, int64_t use_norm, double gain, double eps)
{
    const int64_t half = D / 2;
    double* z = (double*)malloc((size_t)D * sizeof(double));
    double* dz = (double*)malloc((size_t)D * sizeof(double));
    for (int64_t row = 0; row < B * H * T; ++row) {
        const int64_t t = row % T;
        const double* X = x + row * D;
        const double* G = dy + row * D;
        double* DX = dx + row * D;
        for (int64_t i = 0; i < half; ++i) {
            double c = 1.0, s = 0.0;
            if (use_rope) rope_angle(pos0 + t, i, D, base, &c, &s);
            z[i] = X[i] * c - X[i + half] * s;
            z[i + half] = X[i] * s + X[i + half] * c;
        }
        if (use_norm) {
            double ss = 0.0;
            for (int64_t d = 0; d < D; ++d) ss += X[d] * X[d];
            const double rms = sqrt(ss / (double)D + eps);
            double m = 0.0;
            for (int64_t d = 0; d < D; ++d) m += G[d] * z[d];
            m /= (double)D;
            for (int64_t d = 0; d < D; ++d)
                dz[d] = gain / rms * G[d] - z[d] * gain / (rms * rms * rms) * m;
        } else {
            for (int64_t d = 0; d < D; ++d) dz[d] = G[d];
        }
        for (int64_t i = 0; i < half; ++i) {
            double c = 1.0, s = 0.0;
            if (use_rope) rope_angle(pos0 + t, i, D, base, &c, &s);
            DX[i] = dz[i] * c + dz[i + half] * s;
            DX[i + half] = -dz[i] * s + dz[i + half] * c;
        }
    }
    free(z);
    free(dz);
}

/* ------------------------------------------------------------------------ */
/* Pre-norm attention sublayer:  y = x + c_proj(attn(split(c_attn(LN(x)))))  */
/* x, y, dx, dy: [N = B*T][C].  LN weight g[C], bias bl[C].                   */
/* Wa[C][3C], ba[3C] (qkv = u Wa + ba, columns [q | k | v]), Wp[C][C], bp[C]. */
/* Head h of q (and of k, v) is columns h*D .. h*D+D-1 of that third.         */
/* ------------------------------------------------------------------------ */

static void layer_norm_fwd(const double* x, const double* g, const double* bl,
                           double* u, double* xhat, double* rstd, int64_t N,
                           int64_t C, double eps)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double mean = 0.0;
        for (int64_t c = 0; c < C; ++c) mean += x[n * C + c];
        mean /= (double)C;
        double var = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            double t = x[n * C + c] - mean;
            var += t * t;
        }
        var /= (double)C; /* biased variance */
        double r = 1.0 / sqrt(var + eps);
        rstd[n] = r;
        for (int64_t c = 0; c < C; ++c) {
            xhat[n * C + c] = (x[n * C + c] - mean) * r;
            u[n * C + c] = xhat[n * C + c] * g[c] + bl[c];
        }
    }
}

/* Gradient through u = xhat g + bl, xhat = (x - mean) rstd (class LayerNorm,
 * chain rule): dg = sum_n du xhat, dbl = sum_n du, and per row, with
 * dxh = du g, dx = rstd (dxh - mean_c(dxh) - xhat mean_c(dxh xhat)), plus the
 * residual term dres (NULL: none).  xhat, rstd from layer_norm_fwd. */
static void layer_norm_bwd(const double* du, const double* g, const double* xhat,
                           const double* rstd, const double* dres, double* dx, double* dg,
                           double* dbl, int64_t N, int64_t C)
{
    for (int64_t c = 0; c < C; ++c) {
        double ag = 0.0, ab = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            ag += du[n * C + c] * xhat[n * C + c];
            ab += du[n * C + c];
        }
        dg[c] = ag;
        dbl[c] = ab;
    }
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double m1 = 0.0, m2 = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            double dxh = du[n * C + c] * g[c];
            m1 += dxh;
            m2 += dxh * xhat[n * C + c];
        }
        m1 /= (double)C;
        m2 /= (double)C;
        for (int64_t c = 0; c < C; ++c) {
            double dxh = du[n * C + c] * g[c];
            dx[n * C + c] = rstd[n] * (dxh - m1 - xhat[n * C + c] * m2) +
                            (dres ? dres[n * C + c] : 0.0);
        }
    }
}

/* out[N][M] = a[N][Kd] * w[Kd][M] + bias[M] */
static void linear_fwd(const double* a, const double* w, const double* bias,
                       double* out, int64_t N, int64_t Kd, int64_t M)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t j = 0; j < M; ++j) out[n * M + j] = bias[j];
        for (int64_t c = 0; c < Kd; ++c) {
            double av = a[n * Kd + c];
            for (int64_t j = 0; j < M; ++j) out[n * M + j] += av * w[c * M + j];
        }
    }
}

/* [N][3C] columns of one third -> [B][H][T][D] */
static void split_heads(const double* qkv, int64_t third, double* dst,
                        int64_t B, int64_t T, int64_t H, int64_t D)
{
    int64_t C = H * D;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t t = 0; t < T; ++t)
                for (int64_t d = 0; d < D; ++d)
                    dst[((b * H + h) * T + t) * D + d] =
                        qkv[(b * T + t) * 3 * C + third * C + h * D + d];
}

/* [B][H][T][D] -> [N][C] (head merge), optionally into one third of [N][3C] */
static void merge_heads(const double* src, double* dst, int64_t stride,
                        int64_t offset, int64_t B, int64_t T, int64_t H,
                        int64_t D)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t t = 0; t < T; ++t)
                for (int64_t d = 0; d < D; ++d)
                    dst[(b * T + t) * stride + offset + h * D + d] =
                        src[((b * H + h) * T + t) * D + d];
}

typedef struct {
    double *u, *xhat, *rstd, *qkv, *q, *k, *v, *o, *lse, *a;
} sublayer_cache;

static void sublayer_forward_cached(const double* x, const double* g,
                                    const double* bl, const double* Wa,
                                    const double* ba, const double* Wp,
                                    const double* bp, double* y, int64_t B,
                                    int64_t T, int64_t C, int64_t H, double eps,
                                    sublayer_cache* S)
{
    int64_t N = B * T, D = C / H;
    double scale = 1.0 / sqrt((double)D);
    layer_norm_fwd(x, g, bl, S->u, S->xhat, S->rstd, N, C, eps);
    linear_fwd(S->u, Wa, ba, S->qkv, N, C, 3 * C);
    split_heads(S->qkv, 0, S->q, B, T, H, D);
    split_heads(S->qkv, 1, S->k, B, T, H, D);
    split_heads(S->qkv, 2, S->v, B, T, H, D);
    oracle_attn_fwd(S->q, S->k, S->v, S->o, S->lse, B, H, T, D, scale, 0, 0);
    merge_heads(S->o, S->a, C, 0, B, T, H, D);
    linear_fwd(S->a, Wp, bp, y, N, C, C);
    for (int64_t n = 0; n < N * C; ++n) y[n] += x[n];
}

static int cache_alloc(sublayer_cache* S, int64_t N, int64_t C, int64_t H)
{
    S->u = (double*)malloc((size_t)(N * C) * sizeof(double));
    S->xhat = (double*)malloc((size_t)(N * C) * sizeof(double));
    S->rstd = (double*)malloc((size_t)N * sizeof(double));
    S->qkv = (double*)malloc((size_t)(N * 3 * C) * sizeof(double));
    S->q = (double*)malloc((size_t)(N * C) * sizeof(double));
    S->k = (double*)malloc((size_t)(N * C) * sizeof(double));
    S->v = (double*)malloc((size_t)(N * C) * sizeof(double));
    S->o = (double*)malloc((size_t)(N * C) * sizeof(double));
    S->lse = (double*)malloc((size_t)(N * H) * sizeof(double));
    S->a = (double*)malloc((size_t)(N * C) * sizeof(double));
    return S->u && S->xhat && S->rstd && S->qkv && S->q && S->k && S->v &&
           S->o && S->lse && S->a;
}

static void cache_free(sublayer_cache* S)
{
    free(S->u); free(S->xhat); free(S->rstd); free(S->qkv); free(S->q);
    free(S->k); free(S->v); free(S->o); free(S->lse); free(S->a);
}

int oracle_sublayer_fwd(const double* x, const double* g, const double* bl,
                        const double* Wa, const double* ba, const double* Wp,
                        const double* bp, double* y, int64_t B, int64_t T,
                        int64_t C, int64_t H, double eps, int64_t nthreads)
{
    if (H <= 0 || C % H != 0) return 1;
    set_threads(nthreads);
    sublayer_cache S;
    if (!cache_alloc(&S, B * T, C, H)) { cache_free(&S); return 2; }
    sublayer_forward_cached(x, g, bl, Wa, ba, Wp, bp, y, B, T, C, H, eps, &S);
    cache_free(&S);
    return 0;
}

/* Backward of L = sum(dy * y) with respect to x, g, bl, Wa, ba, Wp, bp. */
int oracle_sublayer_bwd(const double* x, const double* g, const double* bl,
                        const double* Wa, const double* ba, const double* Wp,
                        const double* bp, const double* dy, double* dx,
                        double* dg, double* dbl, double* dWa, double* dba,
                        double* dWp, double* dbp, int64_t B, int64_t T,
                        int64_t C, int64_t H, double eps, int64_t nthreads)
{
    if (H <= 0 || C % H != 0) return 1;
    set_threads(nthreads);
    int64_t N = B * T, D = C / H, C3 = 3 * C;
    double scale = 1.0 / sqrt((double)D);
    sublayer_cache S;
    double* y = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* da = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* dO = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* dqh = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* dkh = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* dvh = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* dl = (double*)malloc((size_t)(N * H) * sizeof(double));
    double* dqkv = (double*)malloc((size_t)(N * C3) * sizeof(double));
    double* du = (double*)malloc((size_t)(N * C) * sizeof(double));
    int ok = cache_alloc(&S, N, C, H) && y && da && dO && dqh && dkh && dvh && dl &&
             dqkv && du;
    if (ok) {
        sublayer_forward_cached(x, g, bl, Wa, ba, Wp, bp, y, B, T, C, H, eps, &S);

        /* y = x + a Wp + bp */
        for (int64_t c = 0; c < C; ++c) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += dy[n * C + c];
            dbp[c] = acc;
        }
#pragma omp parallel for schedule(static)
        for (int64_t cp = 0; cp < C; ++cp) {
            /* dWp[cp][c] = sum_n a[n][cp] dy[n][c] */
            for (int64_t c = 0; c < C; ++c) dWp[cp * C + c] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double av = S.a[n * C + cp];
                for (int64_t c = 0; c < C; ++c) dWp[cp * C + c] += av * dy[n * C + c];
            }
        }
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t cp = 0; cp < C; ++cp) {
                double acc = 0.0;
                for (int64_t c = 0; c < C; ++c) acc += dy[n * C + c] * Wp[cp * C + c];
                da[n * C + cp] = acc;
            }

        /* attention, per head */
        for (int64_t b = 0; b < B; ++b)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t t = 0; t < T; ++t)
                    for (int64_t d = 0; d < D; ++d)
                        dO[((b * H + h) * T + t) * D + d] = da[(b * T + t) * C + h * D + d];
        oracle_attn_bwd(S.q, S.k, S.v, dO, dqh, dkh, dvh, dl, B, H, T, D, scale, 0, 0);
        merge_heads(dqh, dqkv, C3, 0, B, T, H, D);
        merge_heads(dkh, dqkv, C3, C, B, T, H, D);
        merge_heads(dvh, dqkv, C3, 2 * C, B, T, H, D);

        /* qkv = u Wa + ba */
        for (int64_t j = 0; j < C3; ++j) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) acc += dqkv[n * C3 + j];
            dba[j] = acc;
        }
#pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < C; ++c) {
            /* dWa[c][j] = sum_n u[n][c] dqkv[n][j] */
            for (int64_t j = 0; j < C3; ++j) dWa[c * C3 + j] = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                double uv = S.u[n * C + c];
                for (int64_t j = 0; j < C3; ++j) dWa[c * C3 + j] += uv * dqkv[n * C3 + j];
            }
        }
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n)
            for (int64_t c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < C3; ++j) acc += dqkv[n * C3 + j] * Wa[c * C3 + j];
                du[n * C + c] = acc;
            }

        /* u = LN(x); the residual path adds dy to dx */
        layer_norm_bwd(du, g, S.xhat, S.rstd, dy, dx, dg, dbl, N, C);
    }
    cache_free(&S);
    free(y); free(da); free(dO); free(dqh); free(dkh); free(dvh); free(dl);
    free(dqkv); free(du);
    return ok ? 0 : 2;
}

/* ------------------------------------------------------------------------ */
/* LayerNorm alone (class LayerNorm of the CS336 tutorial, section 3.4: biased */
/* variance, eps under the square root, gain and bias), its gradient with an  */
/* optional residual term, and the column sums that are a bias's gradient.    */
/* x, y, du, dres, dx: [N][C]; g, bl, dg, dbl: [C].                           */
/* ------------------------------------------------------------------------ */

int oracle_layernorm_fwd(const double* x, const double* g, const double* bl, double* y,
                         int64_t N, int64_t C, double eps, int64_t nthreads)
{
    set_threads(nthreads);
    double* xhat = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* rstd = (double*)malloc((size_t)N * sizeof(double));
    int ok = xhat && rstd;
    if (ok) layer_norm_fwd(x, g, bl, y, xhat, rstd, N, C, eps);
    free(xhat); free(rstd);
    return ok ? 0 : 2;
}

int oracle_layernorm_bwd(const double* x, const double* g, const double* bl, const double* du,
                         const double* dres, double* dx, double* dg, double* dbl, int64_t N,
                         int64_t C, double eps, int64_t nthreads)
{
    set_threads(nthreads);
    double* u = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* xhat = (double*)malloc((size_t)(N * C) * sizeof(double));
    double* rstd = (double*)malloc((size_t)N * sizeof(double));
    int ok = u && xhat && rstd;
    if (ok) {
        layer_norm_fwd(x, g, bl, u, xhat, rstd, N, C, eps);
        layer_norm_bwd(du, g, xhat, rstd, dres, dx, dg, dbl, N, C);
    }
    free(u); free(xhat); free(rstd);
    return ok ? 0 : 2;
}

/* out[j] = sum_n x[n][j]: the gradient of a bias added to every row. */
void oracle_colsum(const double* x, double* out, int64_t N, int64_t M)
{
    for (int64_t j = 0; j < M; ++j) {
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += x[n * M + j];
        out[j] = acc;
    }
}
