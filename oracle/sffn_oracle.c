/*
 * sffn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of the activation-sparse
 * gated FFN forward pass, accumulated in fp64. Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg load it. The HIP library never
 * links, loads or calls it, and the two share no code.
 *
 * What is computed, and where it comes from:
 *   "Model Casting and Low-Parameter Gating: Towards More Sparsely Activated
 *   FFNs" (paper detail page), Abstract: at inference the output of the gating
 *   matrix is computed first; because a sparsity-inducing activation leaves
 *   most of it zero, the products with the two other matrices are skipped for
 *   those channels. LoPA gating gives the gating matrix a low-FLOP
 *   parameterization; here it is the rank-r product W_gate = A.B.
 *   "Mixture-of-Channels: Exploiting Sparse FFNs for Efficient LLMs
 *   Pre-Training and Inference" (blog summary), sections "Dentro il
 *   'mixture'" and "'Dentro MoC'": per token only the Top-K channels of the
 *   SwiGLU gate stay active (a binary mask), and only the weight rows and
 *   columns of active channels are loaded; the same sections and "Kernel e
 *   strutture" name a 2:8 structured-sparsity option. "Model Casting ...",
 *   Abstract, names top-p as a competing sparsification, and the PrunePath
 *   abstract activates units under a cumulative threshold on a
 *   softmax-normalised distribution: the top-p mode reads these at channel
 *   granularity.
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes of the repository):
 *   - the shifted-ReLU gate value is max(z - tau, 0); a channel is active when
 *     z > tau (strict), so z == tau is inactive;
 *   - the Top-K key is the signed SiLU value s = z / (1 + exp(-z)); ties go to
 *     the lower channel index; the gate value of an active channel is s;
 *   - the 2:8 structured option keeps, per token, the 2 largest keys of every
 *     aligned group of 8 consecutive channels, under the same order;
 *   - top-p keeps the shortest prefix of that order whose softmax mass over
 *     the token's keys reaches p;
 *   - the backward runs over the stored active set: the selection passes no
 *     gradient, the shifted ReLU's derivative is 1 on that set, SiLU's is
 *     sigma(z) (1 + z (1 - sigma(z)));
 *   - inputs are the exact values the GPU sees (fp32, or bf16 bit patterns
 *     widened exactly), and every sum runs in ascending index order in fp64.
 *
 * Storage: x [n][d]; W_gate, W_up, W_down [F][d] (row i = channel i);
 * LoPA A^T [r][d] and B^T [F][r]. Element types: 0 = fp32, 1 = bf16 bits,
 * 2 = fp64.
 *
 * Parity of every function here is pinned by the CPU tests (hand-worked
 * examples, textbook special cases, brute force and exact invariants).
 *
 * The OpenMP pragmas only share out independent outputs (channels, columns)
 * for the multi-core timing build; each output is the same sequential sum
 * with or without them, and the plain build ignores them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_F64 = 2 };

/* Read element i of a raw array as fp64. bf16 is the upper half of an IEEE
 * binary32, so shifting the 16-bit pattern up gives the value exactly. */
static inline double elem(const void *base, int dt, long i)
{
    if (dt == OR_F64)
        return ((const double *)base)[i];
    if (dt == OR_F32)
        return (double)((const float *)base)[i];
    uint32_t w = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

void oracle_widen(const void *src, int dt, long count, double *dst)
{
    for (long i = 0; i < count; ++i)
        dst[i] = elem(src, dt, i);
}

/* Gate pre-activation with the full gating matrix: z[t][i] = sum_j x[t][j] Wg[i][j]. */
void oracle_gate_full(int n, int d, int F, const void *x, int x_dt, const void *wg, int w_dt,
                      double *z)
{
    for (int t = 0; t < n; ++t)
#pragma omp parallel for schedule(static)
        for (int i = 0; i < F; ++i) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += elem(x, x_dt, (long)t * d + j) * elem(wg, w_dt, (long)i * d + j);
            z[(long)t * F + i] = acc;
        }
}

/* LoPA gate: t[k] = sum_j x[j] A[j][k] (A stored transposed, [r][d]), then
 * z[i] = sum_k t[k] B[k][i] (B stored transposed, [F][r]). t stays fp64. */
void oracle_gate_lopa(int n, int d, int r, int F, const void *x, int x_dt, const void *at,
                      const void *bt, int w_dt, double *tbuf, double *z)
{
    for (int t = 0; t < n; ++t) {
        double *tv = tbuf + (long)t * r;
#pragma omp parallel for schedule(static)
        for (int k = 0; k < r; ++k) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += elem(x, x_dt, (long)t * d + j) * elem(at, w_dt, (long)k * d + j);
            tv[k] = acc;
        }
#pragma omp parallel for schedule(static)
        for (int i = 0; i < F; ++i) {
            double acc = 0.0;
            for (int k = 0; k < r; ++k)
                acc += tv[k] * elem(bt, w_dt, (long)i * r + k);
            z[(long)t * F + i] = acc;
        }
    }
}

/* Shifted-ReLU gate: g = max(z - tau, 0) for every channel; mask = (z > tau). */
void oracle_select_threshold(int n, int F, const double *z, double tau, unsigned char *mask,
                             double *g)
{
    for (long e = 0; e < (long)n * F; ++e) {
        double v = z[e] - tau;
        mask[e] = z[e] > tau;
        g[e] = v > 0.0 ? v : 0.0;
    }
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

struct keyed {
    double s;
    int i;
};

/* Descending by key, then ascending by channel index: a total order. */
static int keyed_cmp(const void *pa, const void *pb)
{
    const struct keyed *a = (const struct keyed *)pa, *b = (const struct keyed *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->i > b->i) - (a->i < b->i);
}

/* Per-token Top-K of the SiLU gate: g = SiLU(z) for every channel; mask marks
 * the K channels with the largest g (ties to the lower index). kth[t] receives
 * the K-th largest key of token t and nxt[t] the (K+1)-th (-INFINITY when
 * K = F). Returns 0, or -1 on a bad K / no memory. */
int oracle_select_topk(int n, int F, int K, const double *z, unsigned char *mask, double *g,
                       double *kth, double *nxt)
{
    if (K < 1 || K > F) return -1;
    struct keyed *order = (struct keyed *)malloc(sizeof(struct keyed) * (size_t)F);
    if (!order) return -1;
    for (int t = 0; t < n; ++t) {
        const double *zt = z + (long)t * F;
        double *gt = g + (long)t * F;
        unsigned char *mt = mask + (long)t * F;
        for (int i = 0; i < F; ++i) {
            gt[i] = silu(zt[i]);
            order[i].s = gt[i];
            order[i].i = i;
            mt[i] = 0;
        }
        qsort(order, (size_t)F, sizeof(struct keyed), keyed_cmp);
        for (int q = 0; q < K; ++q)
            mt[order[q].i] = 1;
        kth[t] = order[K - 1].s;
        nxt[t] = K < F ? order[K].s : -INFINITY;
    }
    free(order);
    return 0;
}

/* Top-p (cumulative-mass) selection of the SiLU gate: g = SiLU(z) for every
 * channel; each channel's mass is the softmax of the keys over the token,
 * w_i = exp(g_i - max g) / sum_j exp(g_j - max g); in the Top-K order (key
 * descending, then channel ascending) mask keeps the shortest prefix whose
 * mass reaches p (0 < p <= 1). For the parity band: cum[t] = {mass of the
 * prefix without its last channel, mass of the prefix}, and kth[t] / nxt[t]
 * = the last kept and the first dropped key (-INFINITY when none is dropped).
 * Returns 0, or -1 on a bad p / no memory. */
int oracle_select_topp(int n, int F, double p, const double *z, unsigned char *mask, double *g,
                       double *cum, double *kth, double *nxt)
{
    if (!(p > 0.0 && p <= 1.0)) return -1;
    struct keyed *order = (struct keyed *)malloc(sizeof(struct keyed) * (size_t)F);
    if (!order) return -1;
    for (int t = 0; t < n; ++t) {
        const double *zt = z + (long)t * F;
        double *gt = g + (long)t * F;
        unsigned char *mt = mask + (long)t * F;
        double top = -INFINITY;
        for (int i = 0; i < F; ++i) {
            gt[i] = silu(zt[i]);
            order[i].s = gt[i];
            order[i].i = i;
            mt[i] = 0;
            if (gt[i] > top) top = gt[i];
        }
        qsort(order, (size_t)F, sizeof(struct keyed), keyed_cmp);
        double zsum = 0.0;
        for (int q = 0; q < F; ++q)
            zsum += exp(order[q].s - top);
        double c = 0.0, before = 0.0;
        int K = 0;
        while (K < F) {
            before = c;
            c += exp(order[K].s - top) / zsum;
            mt[order[K].i] = 1;
            ++K;
            if (c >= p) break;
        }
        cum[2 * t] = before;
        cum[2 * t + 1] = c;
        kth[t] = order[K - 1].s;
        nxt[t] = K < F ? order[K].s : -INFINITY;
    }
    free(order);
    return 0;
}

/* Structured N:M selection of the SiLU gate (the MoC 2:8 option is N = 2,
 * M = 8): g = SiLU(z) for every channel; the channels are split into aligned
 * groups of M consecutive ones, [M q, M q + M) (the last group may be shorter),
 * and within each group mask marks the N channels with the largest g under
 * the same total order as the Top-K (key descending, then channel ascending);
 * a group of at most N channels keeps them all. bound[t][i] receives the
 * decision boundary of channel i's group, midway between its N-th and
 * (N+1)-th largest keys, or -INFINITY when the group keeps every channel.
 * Returns 0, or -1 on bad N / M or no memory. */
int oracle_select_nm(int n, int F, int N, int M, const double *z, unsigned char *mask, double *g,
                     double *bound)
{
    if (N < 1 || M < N) return -1;
    struct keyed *order = (struct keyed *)malloc(sizeof(struct keyed) * (size_t)M);
    if (!order) return -1;
    for (int t = 0; t < n; ++t) {
        const double *zt = z + (long)t * F;
        double *gt = g + (long)t * F, *bt = bound + (long)t * F;
        unsigned char *mt = mask + (long)t * F;
        for (int q0 = 0; q0 < F; q0 += M) {
            const int len = F - q0 < M ? F - q0 : M;
            for (int e = 0; e < len; ++e) {
                gt[q0 + e] = silu(zt[q0 + e]);
                order[e].s = gt[q0 + e];
                order[e].i = q0 + e;
                mt[q0 + e] = 0;
            }
            qsort(order, (size_t)len, sizeof(struct keyed), keyed_cmp);
            const int keep = len < N ? len : N;
            for (int e = 0; e < keep; ++e)
                mt[order[e].i] = 1;
            const double b = len > N ? 0.5 * (order[N - 1].s + order[N].s) : -INFINITY;
            for (int e = 0; e < len; ++e)
                bt[q0 + e] = b;
        }
    }
    free(order);
    return 0;
}

/* Dense reference: every channel active; act 0 = max(z - tau, 0), act 1 = SiLU(z). */
void oracle_select_dense(int n, int F, int act, const double *z, double tau, unsigned char *mask,
                         double *g)
{
    for (long e = 0; e < (long)n * F; ++e) {
        double v = z[e] - tau;
        mask[e] = 1;
        g[e] = act == 0 ? (v > 0.0 ? v : 0.0) : silu(z[e]);
    }
}

/* Up projection and gating. h[t][i] = mask ? g[t][i] * u[t][i] : 0 with
 * u[t][i] = sum_j x[t][j] Wu[i][j].
 * skip = 0: masked dense (u is formed for every channel, then masked);
 * skip = 1: sparse skip (u is formed only for active channels). */
void oracle_up(int n, int d, int F, const void *x, int x_dt, const void *wu, int w_dt,
               const unsigned char *mask, const double *g, int skip, double *h)
{
    for (int t = 0; t < n; ++t)
#pragma omp parallel for schedule(static)
        for (int i = 0; i < F; ++i) {
            long e = (long)t * F + i;
            if (skip && !mask[e]) {
                h[e] = 0.0;
                continue;
            }
            double u = 0.0;
            for (int j = 0; j < d; ++j)
                u += elem(x, x_dt, (long)t * d + j) * elem(wu, w_dt, (long)i * d + j);
            h[e] = (mask[e] ? 1.0 : 0.0) * g[e] * u;
        }
}

/* Down projection: y[t][c] = sum_i h[t][i] Wd[i][c], i ascending.
 * skip = 0: every channel's row is visited (inactive ones add h = 0);
 * skip = 1: only active channels' rows are visited.
 * Columns are taken in blocks of 64 (one block per thread in an OpenMP
 * build); every y[t][c] is still one sum in ascending i. */
void oracle_down(int n, int d, int F, const double *h, const void *wd, int w_dt,
                 const unsigned char *mask, int skip, double *y)
{
    for (int t = 0; t < n; ++t) {
        double *yt = y + (long)t * d;
#pragma omp parallel for schedule(static)
        for (int c0 = 0; c0 < d; c0 += 64) {
            const int c1 = c0 + 64 < d ? c0 + 64 : d;
            for (int c = c0; c < c1; ++c)
                yt[c] = 0.0;
            for (int i = 0; i < F; ++i) {
                long e = (long)t * F + i;
                if (skip && !mask[e])
                    continue;
                double hv = h[e];
                for (int c = c0; c < c1; ++c)
                    yt[c] += hv * elem(wd, w_dt, (long)i * d + c);
            }
        }
    }
}

/* Union of the per-token active sets: un[i] = OR_t mask[t][i]. Returns |union|. */
int oracle_union(int n, int F, const unsigned char *mask, unsigned char *un)
{
    int count = 0;
    for (int i = 0; i < F; ++i) {
        unsigned char any = 0;
        for (int t = 0; t < n; ++t)
            any |= mask[(long)t * F + i];
        un[i] = any ? 1 : 0;
        count += un[i];
    }
    return count;
}

/* Backward of the layer over a fixed set of active channels ("Mixture-of-
 * Channels" blog summary, "Dentro il 'mixture'": in training only the masked
 * parts are stored and the rest is rebuilt when the backward needs it). With
 * y[t] = sum over active i of g(z[t][i]) u[t][i] Wd[i], z = x.Wg[i],
 * u = x.Wu[i], and dy the gradient of the loss with respect to y, for every
 * active (t, i):
 *   dh = dy[t] . Wd[i]         du = dh g(z)         dz = dh u g'(z)
 *   dWd[i] += g(z) u dy[t]     dWu[i] += du x[t]    dWg[i] += dz x[t]
 *   dx[t]  += du Wu[i] + dz Wg[i]
 * kind 0: g = z - tau, g' = 1 (the shifted ReLU on its active branch; the set
 * says which channels are on); kind 1: g = SiLU(z),
 * g' = sigma(z) (1 + z (1 - sigma(z))). The selection itself is a step
 * function of z and passes no gradient. Every output is overwritten; sums run
 * in ascending token, then channel order, in fp64. */
void oracle_backward(int n, int d, int F, int kind, double tau, const void *x, int x_dt, const void *dy,
                     int dy_dt, const void *wg, const void *wu, const void *wd, int w_dt,
                     const unsigned char *mask, double *dx, double *dwg, double *dwu, double *dwd)
{
    memset(dx, 0, sizeof(double) * (size_t)n * d);
    memset(dwg, 0, sizeof(double) * (size_t)F * d);
    memset(dwu, 0, sizeof(double) * (size_t)F * d);
    memset(dwd, 0, sizeof(double) * (size_t)F * d);
    for (int t = 0; t < n; ++t) {
        for (int i = 0; i < F; ++i) {
            if (!mask[(long)t * F + i])
                continue;
            double z = 0.0, u = 0.0, dh = 0.0;
            for (int k = 0; k < d; ++k) {
                double xv = elem(x, x_dt, (long)t * d + k);
                z += xv * elem(wg, w_dt, (long)i * d + k);
                u += xv * elem(wu, w_dt, (long)i * d + k);
                dh += elem(dy, dy_dt, (long)t * d + k) * elem(wd, w_dt, (long)i * d + k);
            }
            double g, gp;
            if (kind == 0) {
                g = z - tau;
                gp = 1.0;
            } else {
                double sg = 1.0 / (1.0 + exp(-z));
                g = z * sg;
                gp = sg * (1.0 + z * (1.0 - sg));
            }
            double du = dh * g, dz = dh * u * gp, h = g * u;
            for (int k = 0; k < d; ++k) {
                double xv = elem(x, x_dt, (long)t * d + k);
                dwd[(long)i * d + k] += h * elem(dy, dy_dt, (long)t * d + k);
                dwu[(long)i * d + k] += du * xv;
                dwg[(long)i * d + k] += dz * xv;
                dx[(long)t * d + k] += du * elem(wu, w_dt, (long)i * d + k) + dz * elem(wg, w_dt, (long)i * d + k);
            }
        }
    }
}
