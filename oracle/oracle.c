/*
 * oracle.c -- plain, slow, fp64 CPU oracle for exact attention forward and
 * the numerically stable row softmax.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
 * its Python binding) links, loads or calls this file.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header, table or constant with the GPU kernels.
 *
 * Every routine works in IEEE binary64 with plain loops in the order the
 * pages state; no blocking, fusion or reordering is added.  OpenMP only
 * distributes independent rows over threads; the arithmetic of each output
 * element is serial and identical for any thread count.
 *
 * Sources (web pages; title, then the section the code follows):
 *  [L22]  "Lesson 22: why softmax is hard to make efficient, and how
 *         FlashAttention reduces memory traffic" (lincklin.cn).
 *  [FUS]  "Understanding operator fusion through FlashAttention" (jokeuncle).
 *  [GEN]  "Moving less: four generations of FlashAttention" (chengshu-blog).
 *
 * Layouts: Q, K, V, O are contiguous [B][H][N][d] row-major; lse is [B][H][N];
 * x and y of the row softmax are [B][N].  All buffers are host memory owned by
 * the caller.  Return value: 0 on success, -1 on a bad argument, -2 when a
 * scratch allocation fails, -3 when a value has no FP8 code (the encoders).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of OpenMP threads a parallel region here will use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ *
 * Row softmax, three passes over one row ([L22] sections 2 and 3):
 *   pass 1  m = max_j x_j
 *   pass 2  s = sum_j exp(x_j - m)
 *   pass 3  y_j = exp(x_j - m) / s
 * Subtracting the row maximum keeps every exponent <= 0, so no term
 * overflows ([L22] section 2, shift invariance).
 * ------------------------------------------------------------------------ */
static void softmax_row(const double *x, double *y, long n)
{
    double m = -INFINITY;
    for (long j = 0; j < n; ++j)
        if (x[j] > m) m = x[j];
    double s = 0.0;
    for (long j = 0; j < n; ++j)
        s += exp(x[j] - m);
    for (long j = 0; j < n; ++j)
        y[j] = exp(x[j] - m) / s;
}

int oracle_row_softmax(const double *x, double *y, long B, long N)
{
    if (B < 0 || N < 0) return -1;
    if (B == 0 || N == 0) return 0;
    if (!x || !y) return -1;
    long b;
#pragma omp parallel for schedule(dynamic, 16)
    for (b = 0; b < B; ++b)
        softmax_row(x + b * N, y + b * N, N);
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Exact attention for one query row i of one (batch, head) slice, by the
 * three-kernel dataflow that the fused method avoids ([L22] sections 12-14
 * and 25; [FUS] "naive model" and "plain attention dataflow"):
 *   pass 1  s_j = scale * sum_k q_k K_jk  for every key j; under the causal
 *           mask a key j > i is set to -inf without computing its product
 *           ([L22] section 34);
 *   pass 2  m = max_j s_j,  p_j = exp(s_j - m),  l = sum_j p_j,  p_j /= l;
 *   pass 3  o = sum_j p_j V_j,  lse = m + ln l  ([GEN] 2.4: L = m + log l).
 * The score row s and probability row p are materialised in full (n values
 * each).  A row that sees no key (m = -inf) gets o = 0 and lse = -inf; square
 * causal attention never produces one, since key i is visible to query i.
 * ------------------------------------------------------------------------ */
static void attn_row(const double *q, const double *K, const double *V,
                     long n, long d, double scale, long visible,
                     double *s, double *p, double *o, double *lse)
{
    for (long j = 0; j < n; ++j) {
        if (j >= visible) { s[j] = -INFINITY; continue; }
        const double *k = K + j * d;
        double dot = 0.0;
        for (long t = 0; t < d; ++t) dot += q[t] * k[t];
        s[j] = scale * dot;
    }
    double m = -INFINITY;
    for (long j = 0; j < n; ++j)
        if (s[j] > m) m = s[j];
    for (long t = 0; t < d; ++t) o[t] = 0.0;
    if (m == -INFINITY) { *lse = -INFINITY; return; }
    double l = 0.0;
    for (long j = 0; j < n; ++j) {
        p[j] = exp(s[j] - m);      /* exp(-inf) = 0: masked keys get weight 0 */
        l += p[j];
    }
    for (long j = 0; j < n; ++j) p[j] /= l;
    for (long j = 0; j < n; ++j) {
        if (p[j] == 0.0) continue;  /* adds exactly +0.0 to every o[t] */
        const double *v = V + j * d;
        for (long t = 0; t < d; ++t) o[t] += p[j] * v[t];
    }
    *lse = m + log(l);
}

static int attn_args_ok(const void *Q, const void *K, const void *V,
                        const void *O, const void *lse,
                        long B, long H, long N, long d)
{
    if (B < 0 || H < 0 || N < 0 || d < 1) return 0;
    if (B * H * N == 0) return 1;
    return Q && K && V && O && lse;
}

/* Full forward over every (b, h, i): O [B][H][N][d], lse [B][H][N]. */
int oracle_attn_fwd(const double *Q, const double *K, const double *V,
                    double *O, double *lse, long B, long H, long N, long d,
                    double scale, int causal)
{
    if (!attn_args_ok(Q, K, V, O, lse, B, H, N, d)) return -1;
    long total = B * H * N;
    if (total == 0) return 0;
    int failed = 0;
#pragma omp parallel reduction(|| : failed)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *p = (double *)malloc(sizeof(double) * (size_t)N);
        if (!s || !p) {
            failed = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 8)
            for (r = 0; r < total; ++r) {
                long bh = r / N, i = r % N;
                const double *base_k = K + bh * N * d;
                const double *base_v = V + bh * N * d;
                long visible = causal ? i + 1 : N;
                attn_row(Q + r * d, base_k, base_v, N, d, scale, visible,
                         s, p, O + r * d, lse + r);
            }
        }
        free(s);
        free(p);
    }
    return failed ? -2 : 0;
}

/* The same definition for a list of rows only: row r of the output is query
 * index qi[r] of slice bh[r] (bh = b*H + h).  Used where the full tensor is
 * too large for the oracle to finish in seconds; O_rows is [nrows][d]. */
int oracle_attn_rows(const double *Q, const double *K, const double *V,
                     long B, long H, long N, long d, double scale, int causal,
                     const long *bh, const long *qi, long nrows,
                     double *O_rows, double *lse_rows)
{
    if (!attn_args_ok(Q, K, V, O_rows, lse_rows, B, H, N, d) || nrows < 0)
        return -1;
    if (nrows == 0) return 0;
    if (!bh || !qi) return -1;
    for (long r = 0; r < nrows; ++r)
        if (bh[r] < 0 || bh[r] >= B * H || qi[r] < 0 || qi[r] >= N) return -1;
    int failed = 0;
#pragma omp parallel reduction(|| : failed)
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)N);
        double *p = (double *)malloc(sizeof(double) * (size_t)N);
        if (!s || !p) {
            failed = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < nrows; ++r) {
                long slice = bh[r], i = qi[r];
                long visible = causal ? i + 1 : N;
                attn_row(Q + (slice * N + i) * d, K + slice * N * d,
                         V + slice * N * d, N, d, scale, visible,
                         s, p, O_rows + r * d, lse_rows + r);
            }
        }
        free(s);
        free(p);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ *
 * Online softmax over one score row, visited in blocks of bc elements
 * ([L22] sections 18-20 and 33; [GEN] 2.2).  After block t the state is
 *   m_t = max(m_{t-1}, max of block t),
 *   l_t = exp(m_{t-1} - m_t) * l_{t-1} + sum over block t of exp(x - m_t),
 * starting from m_0 = -inf, l_0 = 0.  The state after each block is written
 * to m_trace[t], l_trace[t] (ceil(n / bc) entries each).  The first block
 * would otherwise need exp(-inf - -inf); the correction factor of an empty
 * history (l = 0) is taken as 0 there.
 * ------------------------------------------------------------------------ */
int oracle_online_row_trace(const double *x, long n, long bc,
                            double *m_trace, double *l_trace)
{
    if (n < 0 || bc < 1) return -1;
    if (n == 0) return 0;
    if (!x || !m_trace || !l_trace) return -1;
    double m = -INFINITY, l = 0.0;
    for (long t0 = 0, t = 0; t0 < n; t0 += bc, ++t) {
        long t1 = t0 + bc < n ? t0 + bc : n;
        double block_max = -INFINITY;
        for (long j = t0; j < t1; ++j)
            if (x[j] > block_max) block_max = x[j];
        double m_new = m > block_max ? m : block_max;
        double correction = (m == -INFINITY) ? 0.0 : exp(m - m_new);
        double block_sum = 0.0;
        if (m_new != -INFINITY)
            for (long j = t0; j < t1; ++j) block_sum += exp(x[j] - m_new);
        l = correction * l + block_sum;
        m = m_new;
        m_trace[t] = m;
        l_trace[t] = l;
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Tiled online attention ([L22] sections 21-24 and 32; [GEN] 2.2-2.3 with
 * the deferred normalisation of [GEN] 3.2).  For each block of br query
 * rows the keys are visited in blocks of bc; each row keeps a running
 * maximum m, denominator l and unnormalised output a:
 *   S     = scale * Q_i K_j^T               (masked entries -inf)
 *   m_new = max(m, row max of S)
 *   P     = exp(S - m_new)
 *   c     = exp(m - m_new)
 *   l     = c * l + row sum of P
 *   a     = c * a + P V_j
 *   m     = m_new
 * and at the end o = a / l, lse = m + ln l.  This exists only so the tests
 * can show that the recurrence reaches the three-pass result; it is never
 * compared with the GPU.
 * ------------------------------------------------------------------------ */
int oracle_attn_online(const double *Q, const double *K, const double *V,
                       double *O, double *lse, long B, long H, long N, long d,
                       double scale, int causal, long br, long bc)
{
    if (!attn_args_ok(Q, K, V, O, lse, B, H, N, d) || br < 1 || bc < 1)
        return -1;
    if (B * H * N == 0) return 0;
    long nqb = (N + br - 1) / br;
    long units = B * H * nqb;
    int failed = 0;
#pragma omp parallel reduction(|| : failed)
    {
        double *m = (double *)malloc(sizeof(double) * (size_t)br);
        double *l = (double *)malloc(sizeof(double) * (size_t)br);
        double *a = (double *)malloc(sizeof(double) * (size_t)(br * d));
        double *S = (double *)malloc(sizeof(double) * (size_t)(br * bc));
        if (!m || !l || !a || !S) {
            failed = 1;
        } else {
            long u;
#pragma omp for schedule(dynamic, 1)
            for (u = 0; u < units; ++u) {
                long slice = u / nqb, i0 = (u % nqb) * br;
                long i1 = i0 + br < N ? i0 + br : N, rows = i1 - i0;
                const double *Qs = Q + slice * N * d;
                const double *Ks = K + slice * N * d;
                const double *Vs = V + slice * N * d;
                for (long r = 0; r < rows; ++r) {
                    m[r] = -INFINITY;
                    l[r] = 0.0;
                    for (long t = 0; t < d; ++t) a[r * d + t] = 0.0;
                }
                for (long j0 = 0; j0 < N; j0 += bc) {
                    long j1 = j0 + bc < N ? j0 + bc : N, cols = j1 - j0;
                    for (long r = 0; r < rows; ++r) {
                        long i = i0 + r;
                        for (long c = 0; c < cols; ++c) {
                            long j = j0 + c;
                            if (causal && j > i) { S[r * bc + c] = -INFINITY; continue; }
                            double dot = 0.0;
                            for (long t = 0; t < d; ++t)
                                dot += Qs[i * d + t] * Ks[j * d + t];
                            S[r * bc + c] = scale * dot;
                        }
                        double bmax = -INFINITY;
                        for (long c = 0; c < cols; ++c)
                            if (S[r * bc + c] > bmax) bmax = S[r * bc + c];
                        double m_new = m[r] > bmax ? m[r] : bmax;
                        if (m_new == -INFINITY) continue;  /* nothing visible yet */
                        double corr = (m[r] == -INFINITY) ? 0.0 : exp(m[r] - m_new);
                        double psum = 0.0;
                        for (long t = 0; t < d; ++t) a[r * d + t] *= corr;
                        for (long c = 0; c < cols; ++c) {
                            double pv = exp(S[r * bc + c] - m_new);
                            psum += pv;
                            if (pv == 0.0) continue;
                            const double *v = Vs + (j0 + c) * d;
                            for (long t = 0; t < d; ++t) a[r * d + t] += pv * v[t];
                        }
                        l[r] = corr * l[r] + psum;
                        m[r] = m_new;
                    }
                }
                for (long r = 0; r < rows; ++r) {
                    long idx = slice * N + i0 + r;
                    if (m[r] == -INFINITY) {
                        for (long t = 0; t < d; ++t) O[idx * d + t] = 0.0;
                        lse[idx] = -INFINITY;
                        continue;
                    }
                    for (long t = 0; t < d; ++t) O[idx * d + t] = a[r * d + t] / l[r];
                    lse[idx] = m[r] + log(l[r]);
                }
            }
        }
        free(m);
        free(l);
        free(a);
        free(S);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ *
 * Merge of S partial attention results over disjoint key sets ([L22]
 * section 22: two partial states (m_A, l_A, a_A) and (m_B, l_B, a_B) of one
 * row join as m = max(m_A, m_B), l = e^(m_A - m) l_A + e^(m_B - m) l_B,
 * a = e^(m_A - m) a_A + e^(m_B - m) a_B, and o = a / l; [FUS], the risks
 * list, item 6, for partials kept as accumulated lse and output).
 * Partial s of a row is given normalised, as o_s and lse_s = m_s + ln l_s.
 * Taking lse_s itself as the reference, the same partial is the state
 * (m = lse_s, l = 1, a = o_s); the partials are joined into a running state
 * one after another, s = 0 .. S-1, and the result is o = a / l,
 * lse = m + ln l.  A partial with lse_s = -inf saw no key: it is the empty
 * state and is skipped (its o_s is not read).  A row whose every partial is
 * empty gets o = 0 and lse = -inf.
 *   Opart: [S][rows][d], lpart: [S][rows]; O: [rows][d], lse: [rows].
 * ------------------------------------------------------------------------ */
int oracle_attn_merge(const double *Opart, const double *lpart, double *O,
                      double *lse, long S, long rows, long d)
{
    if (S < 1 || rows < 0 || d < 1) return -1;
    if (rows == 0) return 0;
    if (!Opart || !lpart || !O || !lse) return -1;
    int failed = 0;
#pragma omp parallel reduction(|| : failed)
    {
        double *a = (double *)malloc(sizeof(double) * (size_t)d);
        if (!a) {
            failed = 1;
        } else {
            long r;
#pragma omp for schedule(static)
            for (r = 0; r < rows; ++r) {
                double m = -INFINITY, l = 0.0;
                for (long t = 0; t < d; ++t) a[t] = 0.0;
                for (long s = 0; s < S; ++s) {
                    double m_b = lpart[s * rows + r];
                    if (m_b == -INFINITY) continue;
                    const double *a_b = Opart + (s * rows + r) * d; /* l_b = 1 */
                    double m_new = m > m_b ? m : m_b;
                    double wa = (m == -INFINITY) ? 0.0 : exp(m - m_new);
                    double wb = exp(m_b - m_new);
                    l = wa * l + wb * 1.0;
                    for (long t = 0; t < d; ++t) a[t] = wa * a[t] + wb * a_b[t];
                    m = m_new;
                }
                if (m == -INFINITY) {
                    for (long t = 0; t < d; ++t) O[r * d + t] = 0.0;
                    lse[r] = -INFINITY;
                    continue;
                }
                for (long t = 0; t < d; ++t) O[r * d + t] = a[t] / l;
                lse[r] = m + log(l);
            }
        }
        free(a);
    }
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ *
 * Attention backward: the gradients of the scalar L = sum_{i,t} dO_it O_it
 * with respect to Q, K and V, for the forward above ([L22] sections 30-31
 * and [GEN] 2.4: the probabilities are recomputed from Q and K rather than
 * stored, then dQ, dK, dV follow; the pages do not print the gradient
 * formulas, so they are written out here from the chain rule through
 * O = P V and the row softmax P = softmax(S), S = scale Q K^T with masked
 * entries held at -inf):
 *   dV = P^T dO
 *   dP = dO V^T
 *   D_i = sum_k P_ik dP_ik
 *   dS_ij = P_ij (dP_ij - D_i)            (the softmax Jacobian)
 *   dQ = scale dS K
 *   dK = scale dS^T Q
 * Per (b, h) slice the N x N matrices P and dS are materialised in full; P
 * comes from the three-pass row definition of attn_row.  Rows and columns
 * are distributed over threads; every output element is one serial sum.
 * All tensors are [B][H][N][d].
 * ------------------------------------------------------------------------ */
int oracle_attn_bwd(const double *Q, const double *K, const double *V,
                    const double *dO, double *dQ, double *dK, double *dV,
                    long B, long H, long N, long d, double scale, int causal)
{
    if (!attn_args_ok(Q, K, V, dO, dQ, B, H, N, d) || (B * H * N != 0 && (!dK || !dV)))
        return -1;
    if (B * H * N == 0) return 0;
    double *P = (double *)malloc(sizeof(double) * (size_t)(N * N));
    double *dS = (double *)malloc(sizeof(double) * (size_t)(N * N));
    int failed = (!P || !dS);
    for (long sl = 0; sl < B * H && !failed; ++sl) {
        const double *Qs = Q + sl * N * d, *Ks = K + sl * N * d, *Vs = V + sl * N * d;
        const double *dOs = dO + sl * N * d;
        double *dQs = dQ + sl * N * d, *dKs = dK + sl * N * d, *dVs = dV + sl * N * d;
        int bad = 0;
#pragma omp parallel reduction(|| : bad)
        {
            double *s = (double *)malloc(sizeof(double) * (size_t)N);
            double *o = (double *)malloc(sizeof(double) * (size_t)d);
            if (!s || !o) {
                bad = 1;
            } else {
                long i;
#pragma omp for schedule(dynamic, 8)
                for (i = 0; i < N; ++i) {
                    double lse_i;
                    long visible = causal ? i + 1 : N;
                    attn_row(Qs + i * d, Ks, Vs, N, d, scale, visible, s, P + i * N, o, &lse_i);
                    for (long j = visible; j < N; ++j) P[i * N + j] = 0.0;
                    /* dP_ij = dO_i . V_j, then D_i and dS_ij */
                    double D = 0.0;
                    for (long j = 0; j < N; ++j) {
                        double dp = 0.0;
                        for (long t = 0; t < d; ++t) dp += dOs[i * d + t] * Vs[j * d + t];
                        dS[i * N + j] = dp;
                        D += P[i * N + j] * dp;
                    }
                    for (long j = 0; j < N; ++j) dS[i * N + j] = P[i * N + j] * (dS[i * N + j] - D);
                }
            }
            free(s);
            free(o);
        }
        if (bad) { failed = 1; break; }
        long r;
#pragma omp parallel for schedule(static)
        for (r = 0; r < N; ++r) {
            /* row r of dQ: sum over keys j; row r of dK and dV: sum over queries i */
            for (long t = 0; t < d; ++t) {
                double aq = 0.0, ak = 0.0, av = 0.0;
                for (long j = 0; j < N; ++j) aq += dS[r * N + j] * Ks[j * d + t];
                for (long i = 0; i < N; ++i) {
                    ak += dS[i * N + r] * Qs[i * d + t];
                    av += P[i * N + r] * dOs[i * d + t];
                }
                dQs[r * d + t] = scale * aq;
                dKs[r * d + t] = scale * ak;
                dVs[r * d + t] = av;
            }
        }
    }
    free(P);
    free(dS);
    return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------ *
 * FP8 inputs ([GEN] section 4.6, the FP8 variant: Q, K and V stored as 8-bit
 * floats with a scale per tensor).  The pages name the format but not its
 * encoding; the encoding here is the 8-bit E4M3 one: sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
 * m * 2^-9; exponent field 15 with mantissa 7 is NaN and there are no
 * infinities, so the largest magnitude is 1.75 * 2^8 = 448.
 *   y_i = value(x_i) * s
 * The attention on the decoded values is oracle_attn_fwd itself.
 * ------------------------------------------------------------------------ */
int oracle_fp8_e4m3_decode(const unsigned char *x, double s, double *y, long n)
{
    if (!x || !y || n < 0) return -1;
    for (long i = 0; i < n; ++i) {
        const int sign = x[i] >> 7, e = (x[i] >> 3) & 15, m = x[i] & 7;
        double v;
        if (e == 15 && m == 7)
            v = NAN;
        else if (e == 0)
            v = ldexp((double)m, -9);                 /* subnormal: m / 8 * 2^(1 - 7) */
        else
            v = ldexp(1.0 + (double)m / 8.0, e - 7);  /* normal: 1.m * 2^(e - 7) */
        y[i] = (sign ? -v : v) * s;
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * FP8 encoding: value -> nearest E4M3 code, ties to the even code (the
 * code whose mantissa field is even), sign kept (negative values that round
 * to zero give the code of -0).  The grid is the one oracle_fp8_e4m3_decode
 * reads: normals 1.m * 2^E for E = -6 .. 8 (largest 1.75 * 2^8 = 448),
 * subnormals m * 2^-9.  Encodes x_i / s; returns -3 if some |x_i / s|
 * exceeds 448 or is NaN (no code holds it).
 * ------------------------------------------------------------------------ */
static int fp8_e4m3_encode_one(double x, unsigned char *code)
{
    if (isnan(x)) return -3;
    const int sign = signbit(x) ? 1 : 0;
    const double a = fabs(x);
    if (a > 448.0) return -3;
    int c;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: steps of 2^-9; m = 8 is the smallest normal */
        c = (int)rint(a * 512.0);
    } else {
        int ex;
        frexp(a, &ex);                              /* a = f * 2^ex, f in [0.5, 1) */
        int E = ex - 1;                             /* a = mant * 2^E, mant in [1, 2) */
        int q = (int)rint((ldexp(a, -E) - 1.0) * 8.0);  /* 3 mantissa bits, ties to even */
        if (q == 8) { q = 0; E += 1; }
        c = ((E + 7) << 3) | q;
    }
    *code = (unsigned char)((sign << 7) | c);
    return 0;
}

int oracle_fp8_e4m3_encode(const double *x, double s, unsigned char *out, long n)
{
    if (!x || !out || n < 0 || !(s > 0.0)) return -1;
    for (long i = 0; i < n; ++i)
        if (fp8_e4m3_encode_one(x[i] / s, &out[i]) != 0) return -3;
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Incoherent processing ([GEN] section 4.6): before quantizing, Q and K are
 * both multiplied by one random orthogonal matrix M made of random signs and
 * a Hadamard matrix, which leaves Q K^T unchanged because M M^T = I:
 *   Y = X M,  M = diag(s) H / sqrt(d),
 * H the d x d Hadamard matrix of Sylvester's doubling construction, whose
 * entry (t, k) is (-1)^(number of bits set in both t and k), s_t = +-1.
 * Plain O(d^2) products per row (the pages' O(d log d) fast transform is
 * the kernel's business).  X, Y: [rows][d], d a power of two.
 * ------------------------------------------------------------------------ */
int oracle_hadamard_rotate(const double *X, const double *signs, double *Y, long rows, long d)
{
    if (!X || !signs || !Y || rows < 0 || d <= 0 || (d & (d - 1)) != 0) return -1;
    const double norm = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        const double *x = X + r * d;
        for (long k = 0; k < d; ++k) {
            double acc = 0.0;
            for (long t = 0; t < d; ++t) {
                const int odd = __builtin_popcountl((unsigned long)(t & k)) & 1;
                acc += x[t] * signs[t] * (odd ? -1.0 : 1.0);
            }
            Y[r * d + k] = acc * norm;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ *
 * Block quantization ([GEN] section 4.6: one scale per block instead of one
 * per tensor).  Blocks are 32 consecutive elements along the axis the
 * attention contracts: along a row for Q and K (the head dimension), along
 * the rows of each column for V (the key axis).  A block's scale is a power
 * of two 2^e, stored as the byte e + 127, with e the smallest integer for
 * which the block's largest magnitude amax fits: amax <= 448 * 2^e (e = 0
 * for an all-zero block; the byte is clamped to 0 .. 254).  Each element is
 * the E4M3 code of x / 2^e, and decodes as value(code) * 2^(byte - 127).
 * ------------------------------------------------------------------------ */
static int mx_exponent(double amax)
{
    if (amax == 0.0) return 0;
    int ex;
    frexp(amax, &ex);                                 /* amax < 2^ex */
    int e = ex - 8;                                   /* 448 * 2^(ex - 8) > 2^ex: fits */
    while (amax <= 448.0 * ldexp(1.0, e - 1)) --e;    /* the smallest that fits */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

/* Y [rows][d] -> codes [rows][d], scales [rows][d / 32]; d a multiple of 32. */
int oracle_mx_quantize_rows(const double *Y, unsigned char *codes, unsigned char *scales,
                            long rows, long d)
{
    if (!Y || !codes || !scales || rows < 0 || d <= 0 || d % 32 != 0) return -1;
    int failed = 0;
#pragma omp parallel for schedule(static) reduction(| : failed)
    for (long r = 0; r < rows; ++r)
        for (long blk = 0; blk < d / 32; ++blk) {
            const double *y = Y + r * d + blk * 32;
            double amax = 0.0;
            for (long t = 0; t < 32; ++t)
                if (fabs(y[t]) > amax) amax = fabs(y[t]);
            const int e = mx_exponent(amax);
            scales[r * (d / 32) + blk] = (unsigned char)(e + 127);
            for (long t = 0; t < 32; ++t)
                if (fp8_e4m3_encode_one(ldexp(y[t], -e), &codes[r * d + blk * 32 + t]) != 0)
                    failed = 1;
        }
    return failed ? -3 : 0;
}

/* Y [slices][n][d] -> codes [slices][n][d], scales [slices][ceil(n / 32)][d]:
 * block (i, t) of a slice holds rows 32 i .. min(32 i + 31, n - 1) of
 * column t. */
int oracle_mx_quantize_cols(const double *Y, unsigned char *codes, unsigned char *scales,
                            long slices, long n, long d)
{
    if (!Y || !codes || !scales || slices < 0 || n < 0 || d <= 0) return -1;
    const long nb = (n + 31) / 32;
    int failed = 0;
#pragma omp parallel for schedule(static) reduction(| : failed)
    for (long sl = 0; sl < slices; ++sl)
        for (long i = 0; i < nb; ++i)
            for (long t = 0; t < d; ++t) {
                const long r0 = 32 * i, r1 = (32 * i + 32 < n) ? 32 * i + 32 : n;
                double amax = 0.0;
                for (long r = r0; r < r1; ++r) {
                    const double a = fabs(Y[(sl * n + r) * d + t]);
                    if (a > amax) amax = a;
                }
                const int e = mx_exponent(amax);
                scales[(sl * nb + i) * d + t] = (unsigned char)(e + 127);
                for (long r = r0; r < r1; ++r)
                    if (fp8_e4m3_encode_one(ldexp(Y[(sl * n + r) * d + t], -e),
                                            &codes[(sl * n + r) * d + t]) != 0)
                        failed = 1;
            }
    return failed ? -3 : 0;
}

/* Decoding of the two block layouts: value(code) * 2^(scale byte - 127). */
int oracle_mx_decode_rows(const unsigned char *codes, const unsigned char *scales, double *Y,
                          long rows, long d)
{
    if (!codes || !scales || !Y || rows < 0 || d <= 0 || d % 32 != 0) return -1;
    if (oracle_fp8_e4m3_decode(codes, 1.0, Y, rows * d) != 0) return -1;
    for (long r = 0; r < rows; ++r)
        for (long t = 0; t < d; ++t)
            Y[r * d + t] = ldexp(Y[r * d + t], (int)scales[r * (d / 32) + t / 32] - 127);
    return 0;
}

int oracle_mx_decode_cols(const unsigned char *codes, const unsigned char *scales, double *Y,
                          long slices, long n, long d)
{
    if (!codes || !scales || !Y || slices < 0 || n < 0 || d <= 0) return -1;
    const long nb = (n + 31) / 32;
    if (oracle_fp8_e4m3_decode(codes, 1.0, Y, slices * n * d) != 0) return -1;
    for (long sl = 0; sl < slices; ++sl)
        for (long r = 0; r < n; ++r)
            for (long t = 0; t < d; ++t)
                Y[(sl * n + r) * d + t] =
                    ldexp(Y[(sl * n + r) * d + t], (int)scales[(sl * nb + r / 32) * d + t] - 127);
    return 0;
}
