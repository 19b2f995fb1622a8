/*
 * txl_oracle.c -- CPU oracle for the Transformer-XL relative-attention path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * reference that the HIP library is checked against. It shares no code, header,
 * table or constant with the HIP path, and the product never links or calls it:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark do.
 *
 * Everything is double precision, row-major, with explicit loops. There is no
 * blocking, fusion or shift trick: every score is computed from its own query,
 * key and distance. OpenMP only splits independent outer loops across threads;
 * every sum keeps its sequential order.
 *
 * Sources (web pages on Transformer-XL):
 *  [XL]   "Transformer-XL, explained." (vibeengines.com/paper/transformer-xl):
 *         the seven numbered method steps and the legend of the score equation.
 *  [SIM]  segment-recurrence simulator (mysimulator.uk): the memory equations
 *         h~ = [SG(mem); h], K,V = h~ W, Q = h W, mem = last M rows of h~, and
 *         Attention = softmax(Q K^T / sqrt(d)) V.
 *  [GLO]  Ultralytics glossary "Transformer-XL" (German and Vietnamese): the
 *         segment loop with an empty first memory and the key counts 4, 8.
 *  [IMPL] "Implementing Transformer-XL" (mbrenndoerfer.com): the NumPy layer
 *         with W_q, W_k_E, W_k_R, W_v, W_o, u, v, post-LN residual blocks, the
 *         LayerNorm with population std + 1e-6, and the ReLU FFN.
 *
 * Conventions fixed here where the pages leave them open:
 *  - weights are stored out-major, W[d_out][d_in], and y = x W^T;
 *  - head h owns columns [h*dh, (h+1)*dh) of every D-wide tensor, dh = D/H;
 *  - the distance of query i (segment row) to key j (row of [mem; h]) with m
 *    memory rows is delta = m + i - j; key j is visible iff j <= m + i;
 *  - score = ((q_i + u).k_j + (q_i + v).r_delta) / sqrt(dh), r = R W_kR^T;
 *  - R[delta][k] = sin(delta * 10000^(-2k/D)), R[delta][D/2 + k] = cos(...);
 *  - softmax has no epsilon in the denominator;
 *  - the memory holds the layer's INPUT rows, oldest first.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_NOMEM 2

/* Number of threads the OpenMP loops below use (1 without OpenMP). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the thread count of the OpenMP loops (n >= 1); returns the count in use. */
int orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

/* Relative-encoding table ([XL] step 4 and the legend entry for R_{i-j}).
 * R depends on the distance alone and is not learned; the pages do not print
 * its formula, so the [sin | cos] half-split with base 10000 is the reading
 * taken. D must be even. */
int orc_sinusoid_table(int R_len, int D, double *R)
{
    if (R_len < 0 || D < 2 || (D % 2) != 0 || !R) return ORC_ERR_ARG;
    int half = D / 2;
    for (int d = 0; d < R_len; ++d) {
        for (int k = 0; k < half; ++k) {
            double freq = pow(10000.0, -2.0 * (double)k / (double)D);
            R[(size_t)d * D + k] = sin((double)d * freq);
            R[(size_t)d * D + half + k] = cos((double)d * freq);
        }
    }
    return ORC_OK;
}

/* y[n][o] = sum_i x[n][i] * Wt[o][i]  ([SIM] K,V = h~ W, Q = h W; [IMPL] the
 * projections hidden @ W). */
int orc_linear(long N, int Din, int Dout, const double *x, const double *Wt, double *y)
{
    if (N < 0 || Din < 1 || Dout < 1 || !x || !Wt || !y) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (long n = 0; n < N; ++n) {
        for (int o = 0; o < Dout; ++o) {
            double acc = 0.0;
            for (int i = 0; i < Din; ++i) acc += x[n * Din + i] * Wt[(size_t)o * Din + i];
            y[n * Dout + o] = acc;
        }
    }
    return ORC_OK;
}

/* LayerNorm of [IMPL]: gamma * (x - mean) / (std + 1e-6) + beta, std the
 * population standard deviation over the last axis. */
int orc_layer_norm(long N, int D, const double *x, const double *g, const double *b, double *y)
{
    if (N < 0 || D < 1 || !x || !g || !b || !y) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (long n = 0; n < N; ++n) {
        const double *row = x + n * D;
        double mean = 0.0;
        for (int c = 0; c < D; ++c) mean += row[c];
        mean /= D;
        double var = 0.0;
        for (int c = 0; c < D; ++c) var += (row[c] - mean) * (row[c] - mean);
        var /= D;
        double sd = sqrt(var) + 1e-6;
        for (int c = 0; c < D; ++c) y[n * D + c] = g[c] * (row[c] - mean) / sd + b[c];
    }
    return ORC_OK;
}

/*
 * Relative multi-head attention of one segment over [mem; h] followed by the
 * output projection ([XL] steps 3-4 and the score legend; [SIM]; [IMPL]
 * relative_attention).
 *
 *   h    [B][W][D]   current segment (queries and the last W keys)
 *   mem  [B][m][D]   cached rows, oldest first (ignored when m == 0)
 *   out  [B][W][D]   (P . V) W_o^T
 *   P, AC, BD  optional [B][H][W][m+W]: probabilities (0 where masked), and the
 *              unscaled content and distance terms (NaN where masked).
 */
int orc_rel_attn(int B, int W, int D, int H, int m,
                 const double *h, const double *mem,
                 const double *Wq, const double *WkE, const double *WkR,
                 const double *Wv, const double *Wo,
                 const double *u, const double *v,
                 const double *R, int R_len,
                 double *out, double *P, double *AC, double *BD)
{
    if (B < 1 || W < 1 || D < 1 || H < 1 || D % H != 0 || m < 0) return ORC_ERR_ARG;
    if (!h || (m > 0 && !mem) || !Wq || !WkE || !WkR || !Wv || !Wo || !u || !v || !R || !out)
        return ORC_ERR_ARG;
    const int K = m + W;
    if (R_len < K) return ORC_ERR_ARG;
    const int dh = D / H;
    const double inv_sqrt_dh = 1.0 / sqrt((double)dh);

    /* [SIM] h~ = [SG(mem); h]: memory first, then the segment. */
    double *ctx = malloc(sizeof(double) * (size_t)B * K * D);
    double *Q = malloc(sizeof(double) * (size_t)B * W * D);
    double *KE = malloc(sizeof(double) * (size_t)B * K * D);
    double *V = malloc(sizeof(double) * (size_t)B * K * D);
    double *RK = malloc(sizeof(double) * (size_t)K * D);
    double *O = malloc(sizeof(double) * (size_t)B * W * D);
    if (!ctx || !Q || !KE || !V || !RK || !O) {
        free(ctx); free(Q); free(KE); free(V); free(RK); free(O);
        return ORC_ERR_NOMEM;
    }
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < m; ++j)
            memcpy(ctx + ((size_t)b * K + j) * D, mem + ((size_t)b * m + j) * D, sizeof(double) * D);
        for (int i = 0; i < W; ++i)
            memcpy(ctx + ((size_t)b * K + m + i) * D, h + ((size_t)b * W + i) * D, sizeof(double) * D);
    }

    /* Queries from the segment only; content keys and values from [mem; h]
     * ([XL] step 3); distance keys r = R W_kR^T for every distance 0..K-1
     * ([XL] step 4: separate key projections for content and distance). */
    orc_linear((long)B * W, D, D, h, Wq, Q);
    orc_linear((long)B * K, D, D, ctx, WkE, KE);
    orc_linear((long)B * K, D, D, ctx, Wv, V);
    orc_linear((long)K, D, D, R, WkR, RK);

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int hd = 0; hd < H; ++hd) {
            double *s = malloc(sizeof(double) * K);
            const int c0 = hd * dh;
            for (int i = 0; i < W; ++i) {
                const double *q = Q + ((size_t)b * W + i) * D;
                double smax = -INFINITY;
                for (int j = 0; j < K; ++j) {
                    size_t pidx = (((size_t)b * H + hd) * W + i) * K + j;
                    if (j > m + i) {           /* causal mask over [mem; h] */
                        s[j] = -INFINITY;
                        if (AC) AC[pidx] = NAN;
                        if (BD) BD[pidx] = NAN;
                        continue;
                    }
                    const int delta = m + i - j;   /* query-key distance */
                    const double *k = KE + ((size_t)b * K + j) * D;
                    const double *r = RK + (size_t)delta * D;
                    double ac = 0.0, bd = 0.0;
                    for (int c = c0; c < c0 + dh; ++c) ac += (q[c] + u[c]) * k[c];
                    for (int c = c0; c < c0 + dh; ++c) bd += (q[c] + v[c]) * r[c];
                    if (AC) AC[pidx] = ac;
                    if (BD) BD[pidx] = bd;
                    s[j] = (ac + bd) * inv_sqrt_dh;
                    if (s[j] > smax) smax = s[j];
                }
                double denom = 0.0;
                for (int j = 0; j <= m + i && j < K; ++j) {
                    s[j] = exp(s[j] - smax);
                    denom += s[j];
                }
                for (int j = 0; j < K; ++j) {
                    double p = (j <= m + i) ? s[j] / denom : 0.0;
                    s[j] = p;
                    if (P) P[(((size_t)b * H + hd) * W + i) * K + j] = p;
                }
                double *o = O + ((size_t)b * W + i) * D;
                for (int c = c0; c < c0 + dh; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j < K; ++j) acc += s[j] * V[((size_t)b * K + j) * D + c];
                    o[c] = acc;
                }
            }
            free(s);
        }
    }
    /* Heads concatenated in order, then the output projection ([IMPL]). */
    orc_linear((long)B * W, D, D, O, Wo, out);

    free(ctx); free(Q); free(KE); free(V); free(RK); free(O);
    return ORC_OK;
}

/*
 * Attention with the position encodings Transformer-XL is compared against
 * ([XL] "What it adds to earlier relative positions" and the ablation
 * paragraph of its results; [IMPL] relative_attention's clip of the distance
 * to max_rel_dist), followed by the output projection:
 *
 *   mode ORC_POS_SHAW (Shaw, Uszkoreit and Vaswani): learned embeddings of the
 *     clipped distance, on the keys and on the values, and only the first two
 *     score terms (no u, v):
 *       score_ij = (q_i.k_j + q_i.aK[min(delta, clip)]) / sqrt(dh)
 *       o_i      = sum_j p_ij (val_j + aV[min(delta, clip)])
 *     aK, aV [clip+1][dh], the same tables for every head; delta = m + i - j.
 *   mode ORC_POS_ABSOLUTE: content attention only, score_ij = q_i.k_j / sqrt(dh),
 *     o_i = sum_j p_ij val_j; the positions are already part of the rows
 *     (orc_add_positions on the model's input).
 * Causal over [mem; h] as in orc_rel_attn. Reads Wq, WkE, Wv, Wo.
 */
#define ORC_POS_SHAW 1
#define ORC_POS_ABSOLUTE 2

int orc_attn_variant(int mode, int B, int W, int D, int H, int m,
                     const double *h, const double *mem,
                     const double *Wq, const double *WkE, const double *Wv, const double *Wo,
                     const double *aK, const double *aV, int clip, double *out)
{
    if (mode != ORC_POS_SHAW && mode != ORC_POS_ABSOLUTE) return ORC_ERR_ARG;
    if (B < 1 || W < 1 || D < 1 || H < 1 || D % H != 0 || m < 0) return ORC_ERR_ARG;
    if (!h || (m > 0 && !mem) || !Wq || !WkE || !Wv || !Wo || !out) return ORC_ERR_ARG;
    if (mode == ORC_POS_SHAW && (clip < 0 || !aK || !aV)) return ORC_ERR_ARG;
    const int K = m + W;
    const int dh = D / H;
    const double inv_sqrt_dh = 1.0 / sqrt((double)dh);

    double *ctx = malloc(sizeof(double) * (size_t)B * K * D);
    double *Q = malloc(sizeof(double) * (size_t)B * W * D);
    double *KE = malloc(sizeof(double) * (size_t)B * K * D);
    double *V = malloc(sizeof(double) * (size_t)B * K * D);
    double *O = malloc(sizeof(double) * (size_t)B * W * D);
    if (!ctx || !Q || !KE || !V || !O) {
        free(ctx); free(Q); free(KE); free(V); free(O);
        return ORC_ERR_NOMEM;
    }
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j < m; ++j)
            memcpy(ctx + ((size_t)b * K + j) * D, mem + ((size_t)b * m + j) * D, sizeof(double) * D);
        for (int i = 0; i < W; ++i)
            memcpy(ctx + ((size_t)b * K + m + i) * D, h + ((size_t)b * W + i) * D, sizeof(double) * D);
    }
    orc_linear((long)B * W, D, D, h, Wq, Q);
    orc_linear((long)B * K, D, D, ctx, WkE, KE);
    orc_linear((long)B * K, D, D, ctx, Wv, V);

#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int hd = 0; hd < H; ++hd) {
            double *p = malloc(sizeof(double) * K);
            const int c0 = hd * dh;
            for (int i = 0; i < W; ++i) {
                const double *q = Q + ((size_t)b * W + i) * D;
                const int last = m + i;              /* keys 0..last are visible */
                double smax = -INFINITY;
                for (int j = 0; j <= last; ++j) {
                    const double *k = KE + ((size_t)b * K + j) * D;
                    double sc = 0.0;
                    for (int c = 0; c < dh; ++c) sc += q[c0 + c] * k[c0 + c];
                    if (mode == ORC_POS_SHAW) {
                        const int delta = m + i - j;
                        const double *ak = aK + (size_t)(delta < clip ? delta : clip) * dh;
                        for (int c = 0; c < dh; ++c) sc += q[c0 + c] * ak[c];
                    }
                    p[j] = sc * inv_sqrt_dh;
                    if (p[j] > smax) smax = p[j];
                }
                double denom = 0.0;
                for (int j = 0; j <= last; ++j) {
                    p[j] = exp(p[j] - smax);
                    denom += p[j];
                }
                double *o = O + ((size_t)b * W + i) * D;
                for (int c = 0; c < dh; ++c) {
                    double acc = 0.0;
                    for (int j = 0; j <= last; ++j) {
                        double val = V[((size_t)b * K + j) * D + c0 + c];
                        if (mode == ORC_POS_SHAW) {
                            const int delta = m + i - j;
                            val += aV[(size_t)(delta < clip ? delta : clip) * dh + c];
                        }
                        acc += (p[j] / denom) * val;
                    }
                    o[c0 + c] = acc;
                }
            }
            free(p);
        }
    }
    orc_linear((long)B * W, D, D, O, Wo, out);
    free(ctx); free(Q); free(KE); free(V); free(O);
    return ORC_OK;
}

/*
 * Gradients of relative attention with the memory behind a stop-gradient
 * ([XL] step 2 and the SG(.) legend entry). No gradient reaches the memory
 * rows themselves; gradients flow only through this segment's computation,
 * which includes the projections of the memory rows. Inputs are the
 * projected operands of one segment:
 *   q    [B][W][D]   queries h W_q^T
 *   k    [B][K][D]   content keys of [mem; h] (K = m + W, memory rows first)
 *   val  [B][K][D]   values of [mem; h]
 *   r    [K][D]      distance keys R W_kR^T for distances 0 .. K-1
 *   u, v [D]
 *   dO   [B][W][D]   gradient of the loss w.r.t. the attention output o
 *                    (heads concatenated, before W_o)
 * with score_ij = ((q_i + u).k_j + (q_i + v).r_{m+i-j}) / sqrt(dh), causal, and
 * o_i = sum_j p_ij val_j. Outputs dq [B][W][D], dk, dval [B][K][D], dr [K][D],
 * du, dv [D]: the gradients w.r.t. these operands. Rows j < m of dk and dval
 * belong to the memory's projections (they reach W_kE and W_v); the memory
 * rows themselves are inputs and get no gradient. Per query:
 *   D_i = dO_i . o_i,  dP_ij = dO_i . val_j,  dS_ij = p_ij (dP_ij - D_i)
 *   dq_i += dS_ij (k_j + r_delta) / sqrt(dh),  dk_j += dS_ij (q_i + u) / sqrt(dh)
 *   dval_j += p_ij dO_i,  dr_delta += dS_ij (q_i + v) / sqrt(dh)
 *   du += dS_ij k_j / sqrt(dh),  dv += dS_ij r_delta / sqrt(dh)
 * (the softmax Jacobian applied to dP, then the product rule on each score term).
 * Heads are independent and write disjoint columns, so OpenMP splits heads;
 * within a head every sum runs in (b, i, j) order.
 */
int orc_rel_attn_bwd(int B, int W, int D, int H, int m,
                     const double *q, const double *k, const double *val, const double *r,
                     const double *u, const double *v, const double *dO,
                     double *dq, double *dk, double *dval, double *dr, double *du, double *dv)
{
    if (B < 1 || W < 1 || D < 1 || H < 1 || D % H != 0 || m < 0) return ORC_ERR_ARG;
    if (!q || !k || !val || !r || !u || !v || !dO || !dq || !dk || !dval || !dr || !du || !dv)
        return ORC_ERR_ARG;
    const int K = m + W;
    const int dh = D / H;
    const double c = 1.0 / sqrt((double)dh);
    memset(dq, 0, sizeof(double) * (size_t)B * W * D);
    memset(dk, 0, sizeof(double) * (size_t)B * K * D);
    memset(dval, 0, sizeof(double) * (size_t)B * K * D);
    memset(dr, 0, sizeof(double) * (size_t)K * D);
    memset(du, 0, sizeof(double) * (size_t)D);
    memset(dv, 0, sizeof(double) * (size_t)D);

#pragma omp parallel for schedule(dynamic)
    for (int hd = 0; hd < H; ++hd) {
        const int c0 = hd * dh;
        double *p = malloc(sizeof(double) * K);
        double *ds = malloc(sizeof(double) * K);
        for (int b = 0; b < B; ++b) {
            for (int i = 0; i < W; ++i) {
                const double *qi = q + ((size_t)b * W + i) * D + c0;
                const double *gi = dO + ((size_t)b * W + i) * D + c0;
                const int last = m + i;
                /* forward probabilities of this query */
                double smax = -INFINITY;
                for (int j = 0; j <= last; ++j) {
                    const double *kj = k + ((size_t)b * K + j) * D + c0;
                    const double *rd = r + (size_t)(m + i - j) * D + c0;
                    double sc = 0.0;
                    for (int t = 0; t < dh; ++t) sc += (qi[t] + u[c0 + t]) * kj[t] + (qi[t] + v[c0 + t]) * rd[t];
                    p[j] = sc * c;
                    if (p[j] > smax) smax = p[j];
                }
                double den = 0.0;
                for (int j = 0; j <= last; ++j) { p[j] = exp(p[j] - smax); den += p[j]; }
                for (int j = 0; j <= last; ++j) p[j] /= den;
                /* D_i = dO_i . o_i with o_i = sum_j p_ij val_j */
                double Di = 0.0;
                for (int t = 0; t < dh; ++t) {
                    double o = 0.0;
                    for (int j = 0; j <= last; ++j) o += p[j] * val[((size_t)b * K + j) * D + c0 + t];
                    Di += gi[t] * o;
                }
                for (int j = 0; j <= last; ++j) {
                    const double *vj = val + ((size_t)b * K + j) * D + c0;
                    double dp = 0.0;
                    for (int t = 0; t < dh; ++t) dp += gi[t] * vj[t];
                    ds[j] = p[j] * (dp - Di);
                }
                for (int j = 0; j <= last; ++j) {
                    const int delta = m + i - j;
                    const double *kj = k + ((size_t)b * K + j) * D + c0;
                    const double *rd = r + (size_t)delta * D + c0;
                    double *dqi = dq + ((size_t)b * W + i) * D + c0;
                    double *dkj = dk + ((size_t)b * K + j) * D + c0;
                    double *dvj = dval + ((size_t)b * K + j) * D + c0;
                    double *drd = dr + (size_t)delta * D + c0;
                    for (int t = 0; t < dh; ++t) {
                        dqi[t] += ds[j] * (kj[t] + rd[t]) * c;
                        dkj[t] += ds[j] * (qi[t] + u[c0 + t]) * c;
                        dvj[t] += p[j] * gi[t];
                        drd[t] += ds[j] * (qi[t] + v[c0 + t]) * c;
                        du[c0 + t] += ds[j] * kj[t] * c;
                        dv[c0 + t] += ds[j] * rd[t] * c;
                    }
                }
            }
        }
        free(p);
        free(ds);
    }
    return ORC_OK;
}

/* Absolute positions of the ablation ([XL] results: absolute encodings with
 * recurrence): y[b][t] = x[b][t] + U[pos0 + t], U the sinusoid of orc_sinusoid_table
 * evaluated at the absolute position instead of a distance. */
int orc_add_positions(int B, int W, int D, int pos0, const double *x, double *y)
{
    if (B < 1 || W < 1 || D < 2 || D % 2 || pos0 < 0 || !x || !y) return ORC_ERR_ARG;
    double *U = malloc(sizeof(double) * (size_t)(pos0 + W) * D);
    if (!U) return ORC_ERR_NOMEM;
    orc_sinusoid_table(pos0 + W, D, U);
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < W; ++t)
            for (int c = 0; c < D; ++c)
                y[((size_t)b * W + t) * D + c] = x[((size_t)b * W + t) * D + c] + U[(size_t)(pos0 + t) * D + c];
    free(U);
    return ORC_OK;
}

/* Post-LN block of [IMPL] forward: h1 = LN1(h + attn), y = LN2(h1 + FFN(h1)),
 * FFN(x) = ReLU(x W1^T + b1) W2^T + b2. */
int orc_layer_fwd(int B, int W, int D, int H, int F, int m,
                  const double *h, const double *mem,
                  const double *Wq, const double *WkE, const double *WkR,
                  const double *Wv, const double *Wo,
                  const double *u, const double *v,
                  const double *ln1_g, const double *ln1_b,
                  const double *W1, const double *b1, const double *W2, const double *b2,
                  const double *ln2_g, const double *ln2_b,
                  const double *R, int R_len, double *y)
{
    if (F < 1 || !ln1_g || !ln1_b || !W1 || !b1 || !W2 || !b2 || !ln2_g || !ln2_b || !y)
        return ORC_ERR_ARG;
    const long N = (long)B * W;
    double *att = malloc(sizeof(double) * N * D);
    double *h1 = malloc(sizeof(double) * N * D);
    double *f1 = malloc(sizeof(double) * N * F);
    double *f2 = malloc(sizeof(double) * N * D);
    if (!att || !h1 || !f1 || !f2) { free(att); free(h1); free(f1); free(f2); return ORC_ERR_NOMEM; }
    int st = orc_rel_attn(B, W, D, H, m, h, mem, Wq, WkE, WkR, Wv, Wo, u, v, R, R_len,
                          att, NULL, NULL, NULL);
    if (st != ORC_OK) { free(att); free(h1); free(f1); free(f2); return st; }
    for (long n = 0; n < N * D; ++n) att[n] += h[n];
    orc_layer_norm(N, D, att, ln1_g, ln1_b, h1);
    orc_linear(N, D, F, h1, W1, f1);
    for (long n = 0; n < N; ++n)
        for (int c = 0; c < F; ++c) {
            double z = f1[n * F + c] + b1[c];
            f1[n * F + c] = z > 0.0 ? z : 0.0;
        }
    orc_linear(N, F, D, f1, W2, f2);
    for (long n = 0; n < N; ++n)
        for (int c = 0; c < D; ++c) f2[n * D + c] += b2[c] + h1[n * D + c];
    orc_layer_norm(N, D, f2, ln2_g, ln2_b, y);
    free(att); free(h1); free(f1); free(f2);
    return ORC_OK;
}

/* Memory update of [SIM]: mem <- last M rows of h~ = [mem; h] (logical order,
 * oldest first). new_mem must hold [B][M][D]; returns the new row count. */
int orc_mem_update(int B, int M, int D, int m, const double *mem, int W, const double *h,
                   double *new_mem, int *new_m)
{
    if (B < 1 || M < 1 || D < 1 || m < 0 || m > M || W < 1 || !h || !new_mem || !new_m)
        return ORC_ERR_ARG;
    const int K = m + W;
    const int keep = K < M ? K : M;
    for (int b = 0; b < B; ++b) {
        for (int t = 0; t < keep; ++t) {
            int src = K - keep + t;   /* row of [mem; h] */
            const double *row = src < m ? mem + ((size_t)b * m + src) * D
                                        : h + ((size_t)b * W + (src - m)) * D;
            memcpy(new_mem + ((size_t)b * M + t) * D, row, sizeof(double) * D);
        }
    }
    *new_m = keep;
    return ORC_OK;
}

/*
 * Segment-by-segment driver over a stream x [B][S*W][D] ([XL] steps 1-3 and 6:
 * segments in order, every layer caches its input rows, layer n reads the
 * cache of layer n-1's states). Layer parameters are stacked along a leading
 * axis of size L. full_layer = 0 runs the attention + output projection only
 * (single-layer attention workloads); full_layer = 1 runs the post-LN block.
 * The memory of every layer starts empty, or, when mems_in ([L][B][M][D],
 * oldest row first) and mem_len_in ([L]) are given, holds those rows (a stream
 * resumed after earlier segments). y [B][S*W][D] receives the last layer's
 * output per segment; mems_out (optional, [L][B][M][D]) and mem_len_out
 * (optional, [L]) receive the final memories in the same form.
 */
int orc_stack_fwd(int B, int W, int D, int H, int F, int L, int S, int M, int full_layer,
                  const double *x,
                  const double *Wq, const double *WkE, const double *WkR,
                  const double *Wv, const double *Wo,
                  const double *u, const double *v,
                  const double *ln1_g, const double *ln1_b,
                  const double *W1, const double *b1, const double *W2, const double *b2,
                  const double *ln2_g, const double *ln2_b,
                  const double *R, int R_len, double *y, double *mems_out, int *mem_len_out,
                  const double *mems_in, const int *mem_len_in)
{
    if (B < 1 || W < 1 || D < 1 || H < 1 || L < 1 || S < 1 || M < 1 || !x || !y) return ORC_ERR_ARG;
    if (full_layer && F < 1) return ORC_ERR_ARG;
    if ((mems_in == NULL) != (mem_len_in == NULL)) return ORC_ERR_ARG;
    if (mem_len_in)
        for (int l = 0; l < L; ++l)
            if (mem_len_in[l] < 0 || mem_len_in[l] > M) return ORC_ERR_ARG;
    const size_t DD = (size_t)D * D;
    const size_t seg = (size_t)W * D;
    double *mems = calloc((size_t)L * B * M * D, sizeof(double));
    double *tmp_mem = calloc((size_t)B * M * D, sizeof(double));
    int *mlen = calloc((size_t)L, sizeof(int));
    double *hin = malloc(sizeof(double) * (size_t)B * seg);
    double *hout = malloc(sizeof(double) * (size_t)B * seg);
    if (!mems || !tmp_mem || !mlen || !hin || !hout) {
        free(mems); free(tmp_mem); free(mlen); free(hin); free(hout);
        return ORC_ERR_NOMEM;
    }
    /* a stream resumed from carried memories (same [L][B][M][D] layout and
     * lengths as mems_out / mem_len_out): the memory is the only state that
     * crosses a segment boundary, so nothing else is needed */
    if (mems_in) {
        memcpy(mems, mems_in, sizeof(double) * (size_t)L * B * M * D);
        memcpy(mlen, mem_len_in, sizeof(int) * (size_t)L);
    }
    int st = ORC_OK;
    for (int t = 0; t < S && st == ORC_OK; ++t) {
        for (int b = 0; b < B; ++b)
            memcpy(hin + (size_t)b * seg, x + ((size_t)b * S + t) * seg, sizeof(double) * seg);
        for (int l = 0; l < L && st == ORC_OK; ++l) {
            const int m = mlen[l];
            /* the memory buffer holds [B][M][D]; pass its first m rows per batch
             * as a compact [B][m][D] block */
            double *mcompact = malloc(sizeof(double) * (size_t)B * (m > 0 ? m : 1) * D);
            for (int b = 0; b < B; ++b)
                memcpy(mcompact + (size_t)b * m * D, mems + (((size_t)l * B + b) * M) * D,
                       sizeof(double) * (size_t)m * D);
            if (full_layer)
                st = orc_layer_fwd(B, W, D, H, F, m, hin, mcompact,
                                   Wq + l * DD, WkE + l * DD, WkR + l * DD, Wv + l * DD, Wo + l * DD,
                                   u + (size_t)l * D, v + (size_t)l * D,
                                   ln1_g + (size_t)l * D, ln1_b + (size_t)l * D,
                                   W1 + (size_t)l * F * D, b1 + (size_t)l * F,
                                   W2 + (size_t)l * D * F, b2 + (size_t)l * D,
                                   ln2_g + (size_t)l * D, ln2_b + (size_t)l * D,
                                   R, R_len, hout);
            else
                st = orc_rel_attn(B, W, D, H, m, hin, mcompact,
                                  Wq + l * DD, WkE + l * DD, WkR + l * DD, Wv + l * DD, Wo + l * DD,
                                  u + (size_t)l * D, v + (size_t)l * D, R, R_len,
                                  hout, NULL, NULL, NULL);
            if (st == ORC_OK) {
                int nm = 0;
                /* the layer's input rows go to its memory */
                st = orc_mem_update(B, M, D, m, mcompact, W, hin, tmp_mem, &nm);
                memcpy(mems + (size_t)l * B * M * D, tmp_mem, sizeof(double) * (size_t)B * M * D);
                mlen[l] = nm;
            }
            free(mcompact);
            double *sw = hin; hin = hout; hout = sw;   /* next layer's input */
        }
        for (int b = 0; b < B; ++b)
            memcpy(y + ((size_t)b * S + t) * seg, hin + (size_t)b * seg, sizeof(double) * seg);
    }
    if (mems_out) memcpy(mems_out, mems, sizeof(double) * (size_t)L * B * M * D);
    if (mem_len_out) memcpy(mem_len_out, mlen, sizeof(int) * (size_t)L);
    free(mems); free(tmp_mem); free(mlen); free(hin); free(hout);
    return st;
}
