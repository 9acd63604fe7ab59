/*
 * dfp_oracle.c -- plain fp64 CPU oracle for displaced patch attention and the
 * per-step guidance / sampler / rel-MAE computation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library: every quantity is recomputed here from the definitions on
 * the pages, in double precision, with no blocking, fusion or reordering
 * beyond what the definition states.
 *
 * Sources (page title, section):
 *   [DF]  "终极性能对比：DistriFusion vs 传统推理方案", section
 *         "DistriFusion的革命性突破": first steps synchronous, later steps
 *         reuse activations of the previous step.
 *   [XD]  "xDiT: an Inference Engine for Diffusion Transformers (DiTs) with
 *         Massive Parallelism", section 三.2 PipeFusion (M non-overlapping
 *         patches) and 三.3 CFG Parallelism (cond/uncond = a batch of 2).
 *   [HY]  "Accelerating Diffusion via Hybrid Data-Pipeline Parallelism Based
 *         on Conditional Guidance Scheduling", section 关键设计 2 (rel-MAE of
 *         the two noise predictions, an L1 ratio with the unconditional term
 *         below) and 损失函数/训练策略 (flow matching: swap eps for v).
 *   [AI]  "AIGC 文生图系统如何优化扩散模型推理速度", section 1 (x_T drawn
 *         from N(0,1)) and section 3 (DDIM with eta; eta = 0 deterministic).
 *   [DT]  "DistriFusion高级教程：自定义并行配置实现超高清图像生成的完整指南",
 *         sections 多设备配置优化 and 速度与质量平衡: a communication mode
 *         named corrected_async_gn (an asynchronous GroupNorm with a
 *         correction), given by name only.
 *
 * Readings taken where the pages are silent:
 *   - attention is plain softmax(Q K^T * scale) V with no mask or bias;
 *   - the CFG combine is g = g_u + w (g_c - g_u)  (not printed on [XD]/[HY]);
 *   - DDIM's undefined sigma_t in x0_hat is sqrt(1 - abar_t);
 *   - "scaled linear" betas are linear in sqrt(beta);
 *   - the flow sampler is plain Euler on sigma_i = 1 - i/S;
 *   - corrected_async_gn: GroupNorm whose per-group statistics come from
 *     every other patch's partial sums of the previous step (stale, as [DF]
 *     reuses activations) plus this patch's own sums of this step (fresh:
 *     the correction), over equal-size patches; statistics are the plain
 *     mean and biased variance of the group, eps inside the square root.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* The persistent K/V buffer after the fresh patch rows have landed.          */
/* [DF] later steps attend over the previous step's activations everywhere   */
/* except the local patch, whose activations are this step's.  [XD] 三.2:    */
/* a patch is one of M non-overlapping token ranges.                          */
/* buf: [BH][N][d] stale rows (overwritten in place); fresh: [BH][n][d].     */
/* ------------------------------------------------------------------------ */
void oracle_effective_kv(double *buf, const double *fresh, int64_t BH, int64_t N,
                         int64_t d, int64_t row0, int64_t n)
{
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t i = 0; i < n; ++i)
            for (int64_t c = 0; c < d; ++c)
                buf[(bh * N + row0 + i) * d + c] = fresh[(bh * n + i) * d + c];
}

/* ------------------------------------------------------------------------ */
/* One query row of attention over N_kv keys, two passes, no online          */
/* rescaling:  s_j = scale * <q, k_j>;  m = max_j s_j;  p_j = exp(s_j - m);  */
/* l = sum_j p_j;  o = sum_j p_j v_j / l.                                     */
/* scratch must hold N_kv doubles.                                            */
/* ------------------------------------------------------------------------ */
static void attention_row(const double *q, const double *k, const double *v,
                          int64_t Nkv, int64_t d, double scale, double *o,
                          double *s)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < Nkv; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c)
            dot += q[c] * k[j * d + c];
        s[j] = scale * dot;
        if (s[j] > m)
            m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < Nkv; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    for (int64_t c = 0; c < d; ++c)
        o[c] = 0.0;
    for (int64_t j = 0; j < Nkv; ++j)
        for (int64_t c = 0; c < d; ++c)
            o[c] += s[j] * v[j * d + c];
    for (int64_t c = 0; c < d; ++c)
        o[c] /= l;
}

/* Attention for every query row of every (batch, head).
 * q: [BH][nq][d], k, v: [BH][Nkv][d] (already the effective buffer),
 * o: [BH][nq][d].  Returns 0, or -1 if scratch could not be allocated. */
int oracle_attention(const double *q, const double *k, const double *v,
                     int64_t BH, int64_t nq, int64_t Nkv, int64_t d,
                     double scale, double *o)
{
    int failed = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nkv > 0 ? Nkv : 1));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for collapse(2) schedule(dynamic, 4)
            for (int64_t bh = 0; bh < BH; ++bh)
                for (int64_t i = 0; i < nq; ++i)
                    attention_row(q + (bh * nq + i) * d, k + bh * Nkv * d,
                                  v + bh * Nkv * d, Nkv, d, scale,
                                  o + (bh * nq + i) * d, s);
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* Attention for a chosen subset of (bh, row) pairs, for sampled checks at
 * sizes where every row would take too long.  rows_bh[r], rows_i[r] name the
 * r-th row; o: [nrows][d]. */
int oracle_attention_rows(const double *q, const double *k, const double *v,
                          int64_t BH, int64_t nq, int64_t Nkv, int64_t d,
                          double scale, const int64_t *rows_bh,
                          const int64_t *rows_i, int64_t nrows, double *o)
{
    int failed = 0;
    (void)BH;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Nkv > 0 ? Nkv : 1));
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t bh = rows_bh[r], i = rows_i[r];
                attention_row(q + (bh * nq + i) * d, k + bh * Nkv * d,
                              v + bh * Nkv * d, Nkv, d, scale, o + r * d, s);
            }
            free(s);
        }
    }
    return failed ? -1 : 0;
}

/* The softmax probability matrix itself, for tiny inputs: p: [BH][nq][Nkv]. */
void oracle_attention_probs(const double *q, const double *k, int64_t BH,
                            int64_t nq, int64_t Nkv, int64_t d, double scale,
                            double *p)
{
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t i = 0; i < nq; ++i) {
            const double *qi = q + (bh * nq + i) * d;
            double *row = p + (bh * nq + i) * Nkv;
            double m = -INFINITY;
            for (int64_t j = 0; j < Nkv; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += qi[c] * k[(bh * Nkv + j) * d + c];
                row[j] = scale * dot;
                if (row[j] > m)
                    m = row[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < Nkv; ++j) {
                row[j] = exp(row[j] - m);
                l += row[j];
            }
            for (int64_t j = 0; j < Nkv; ++j)
                row[j] /= l;
        }
}

/* ------------------------------------------------------------------------ */
/* Noise schedule.  [AI] section 3 asks the schedule for alpha_t and the     */
/* cumulative alpha-bar_t; the workload names a 1000-step "scaled linear"    */
/* schedule from 0.00085 to 0.012, read as linear in sqrt(beta):             */
/*   beta_i = (sqrt(b0) + (sqrt(b1) - sqrt(b0)) * i / (T-1))^2               */
/*   abar_t = prod_{i<=t} (1 - beta_i).                                      */
/* ------------------------------------------------------------------------ */
void oracle_scaled_linear_betas(int64_t T, double beta_start, double beta_end,
                                double *beta)
{
    double a = sqrt(beta_start), b = sqrt(beta_end);
    for (int64_t i = 0; i < T; ++i) {
        double r = a + (b - a) * (double)i / (double)(T - 1);
        beta[i] = r * r;
    }
}

void oracle_alphas_cumprod(int64_t T, const double *beta, double *abar)
{
    double prod = 1.0;
    for (int64_t t = 0; t < T; ++t) {
        prod *= (1.0 - beta[t]);
        abar[t] = prod;
    }
}

/* [AI] section 3: the sampled timesteps are linspace(0, T-1, S) rounded to
 * integers (numpy's round: halves go to the even neighbour), then walked in
 * reverse.  ts receives the ascending sequence. */
void oracle_ddim_timesteps(int64_t T, int64_t S, int64_t *ts)
{
    for (int64_t i = 0; i < S; ++i) {
        double x = (S == 1) ? 0.0 : (double)(T - 1) * (double)i / (double)(S - 1);
        ts[i] = (int64_t)nearbyint(x); /* default rounding mode: ties to even */
    }
}

/* ------------------------------------------------------------------------ */
/* Classifier-free guidance.  [XD] 三.3 and [HY] 关键设计 1: the guided       */
/* prediction is formed from a conditional and an unconditional pass over   */
/* the same x_t.  The combine is read as g = g_u + w (g_c - g_u).            */
/* ------------------------------------------------------------------------ */
void oracle_cfg_combine(const double *g_c, const double *g_u, int64_t n,
                        double w, double *g)
{
    for (int64_t i = 0; i < n; ++i)
        g[i] = g_u[i] + w * (g_c[i] - g_u[i]);
}

/* [AI] section 3, DDIM.  The DDIM update moves x_t to the previous sampled
 * timestep in three parts, all read off the noise prediction eps:
 *   the predicted clean latent   x0  = (x_t - sqrt(1 - abar_t) eps) / sqrt(abar_t)
 *     (the page's undefined sigma_t is read as sqrt(1 - abar_t));
 *   the direction back to x_t    dir = sqrt(1 - abar_prev - sigma^2) eps;
 *   fresh noise                  sigma z,  z ~ N(0, 1);
 * and x_{t-1} = sqrt(abar_prev) x0 + dir + sigma z.  The page's final step
 * returns x0 itself, which is this update with abar_prev = 1 (then sigma = 0
 * and dir = 0).  sigma is the step's noise scale, see oracle_ddim_sigma. */
double oracle_ddim_sigma(double abar_t, double abar_prev, double eta)
{
    /* [AI] section 3: eta scales the standard deviation of the DDPM
     * posterior q(x_{t-1} | x_t, x0); eta = 0 is deterministic DDIM. */
    double posterior_var = (1.0 - abar_prev) / (1.0 - abar_t) * (1.0 - abar_t / abar_prev);
    return eta * sqrt(posterior_var);
}

void oracle_ddim_update(double *x, const double *eps, const double *z, int64_t n,
                        double abar_t, double abar_prev, double sigma)
{
    const double keep = sqrt(abar_prev);                           /* on x0  */
    const double toward = sqrt(1.0 - abar_prev - sigma * sigma);   /* on eps */
    for (int64_t i = 0; i < n; ++i) {
        double pred_x0 = (x[i] - sqrt(1.0 - abar_t) * eps[i]) / sqrt(abar_t);
        double noise = (z != NULL) ? sigma * z[i] : 0.0;
        x[i] = keep * pred_x0 + toward * eps[i] + noise;
    }
}

/* ------------------------------------------------------------------------ */
/* The standard-normal draw z of a DDIM step with eta > 0 ([AI] section 3    */
/* draws it with randn_like).  To draw the same z on any device it comes     */
/* from a counter-based generator: Philox4x64 with 10 rounds (J. Salmon,     */
/* M. Moraes, R. Dror, D. Shaw, "Parallel Random Numbers: As Easy as 1, 2,   */
/* 3", SC'11), followed by the Box-Muller transform (G. Box, M. Muller, "A   */
/* Note on the Generation of Random Normal Deviates", 1958).                 */
/* ------------------------------------------------------------------------ */

/* One Philox4x64-10 block.  Each round multiplies counter words 0 and 2 by
 * the round constants (full 128-bit products), and the new counter is
 * (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); between
 * rounds the key is advanced by the two Weyl constants. */
void oracle_philox4x64_10(const uint64_t ctr[4], const uint64_t key[2], uint64_t out[4])
{
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    uint64_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint64_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        unsigned __int128 p0 = (unsigned __int128)M0 * c0;
        unsigned __int128 p1 = (unsigned __int128)M1 * c2;
        uint64_t n0 = (uint64_t)(p1 >> 64) ^ c1 ^ k0;
        uint64_t n1 = (uint64_t)p1;
        uint64_t n2 = (uint64_t)(p0 >> 64) ^ c3 ^ k1;
        uint64_t n3 = (uint64_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* z[0..n) of image `image` at sampler step `step` under `seed`.  Block j
 * (elements 8j .. 8j+7) is Philox4x64-10 of counter (j, image, 0, 0) under
 * key (seed, step).  Its four 64-bit words give eight 32-bit halves h_0..h_7
 * (h_{2k} the low half of word k, h_{2k+1} the high half), each mapped to a
 * uniform u = (h + 1/2) / 2^32 in (0, 1).  Pair k turns (u_{2k}, u_{2k+1})
 * into two normals by Box-Muller:
 *   z[8j+2k]   = sqrt(-2 ln u_{2k}) cos(2 pi u_{2k+1})
 *   z[8j+2k+1] = sqrt(-2 ln u_{2k}) sin(2 pi u_{2k+1}). */
void oracle_philox_normals(double *z, int64_t n, uint64_t seed, uint64_t step, uint64_t image)
{
    const double two_pi = 6.283185307179586476925286766559;
    const uint64_t key[2] = {seed, step};
    for (int64_t j = 0; 8 * j < n; ++j) {
        const uint64_t ctr[4] = {(uint64_t)j, image, 0, 0};
        uint64_t w[4];
        oracle_philox4x64_10(ctr, key, w);
        double u[8];
        for (int k = 0; k < 4; ++k) {
            u[2 * k] = ((double)(w[k] & 0xFFFFFFFFull) + 0.5) / 4294967296.0;
            u[2 * k + 1] = ((double)(w[k] >> 32) + 0.5) / 4294967296.0;
        }
        for (int k = 0; k < 4; ++k) {
            double r = sqrt(-2.0 * log(u[2 * k]));
            double a = two_pi * u[2 * k + 1];
            if (8 * j + 2 * k < n) z[8 * j + 2 * k] = r * cos(a);
            if (8 * j + 2 * k + 1 < n) z[8 * j + 2 * k + 1] = r * sin(a);
        }
    }
}

/* Run a parallel region of this library on `threads` threads from now on
 * (harness plumbing for timing the oracle on one core; no arithmetic). */
void oracle_set_threads(int threads)
{
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
}

/* [HY] 损失函数/训练策略: flow-matching models predict a velocity v in place
 * of eps.  Integrator (not on the pages): Euler on sigma,
 *   x <- x + (sigma_next - sigma) * v,  sigma_i = 1 - i/S, i = 0..S. */
void oracle_flow_sigmas(int64_t S, double *sigma)
{
    for (int64_t i = 0; i <= S; ++i)
        sigma[i] = 1.0 - (double)i / (double)S;
}

void oracle_euler_step(double *x, const double *v, int64_t n, double sigma,
                       double sigma_next)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = x[i] + (sigma_next - sigma) * v[i];
}

/* [HY] 关键设计 2: the denoising discrepancy is the relative mean absolute
 * error of the two predictions; with the unconditional prediction as the
 * reference it is sum |g_c - g_u| / sum |g_u| over one image.  IEEE division
 * decides the degenerate cases (0/0 = NaN, x/0 = +Inf). */
double oracle_relmae(const double *g_c, const double *g_u, int64_t n)
{
    double num = 0.0, den = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        num += fabs(g_c[i] - g_u[i]);
        den += fabs(g_u[i]);
    }
    return num / den;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* [HY] 关键设计 3 (adaptive switching over the rel-MAE curve): with M_t the
 * denoising discrepancy of step t (t = 0 the first, noisiest step),
 *   G_t      = (M_t - M_{t-L}) / L                 for t >= L
 *   tau1'    = min { t : 0 <= G_t < g_slope }      (undefined if no such t)
 *   tau_cap  = the step of the curve's global minimum (first on ties)
 *   tau1     = min(tau1', tau_cap)   (tau_cap alone when tau1' is undefined)
 *   tau2     = tau1 + k,  clamped to S (no fully-connecting phase then).
 * Warm-up is steps [0, tau1], parallel (tau1, tau2), fully-connecting
 * [tau2, S).  Returns 0, or -1 for S < 1 or L < 1. */
int oracle_switch_points(const double *M, int64_t S, int64_t L, double g_slope, int64_t k,
                         int64_t *tau1, int64_t *tau2)
{
    if (S < 1 || L < 1) return -1;
    int64_t cap = 0;
    for (int64_t t = 1; t < S; ++t)
        if (M[t] < M[cap]) cap = t;
    int64_t first = -1;
    for (int64_t t = L; t < S; ++t) {
        double G = (M[t] - M[t - L]) / (double)L;
        if (G >= 0.0 && G < g_slope) {
            first = t;
            break;
        }
    }
    int64_t t1 = (first >= 0 && first < cap) ? first : cap;
    int64_t t2 = t1 + k;
    if (t2 > S) t2 = S;
    *tau1 = t1;
    *tau2 = t2;
    return 0;
}


/* ------------------------------------------------------------------------ */
/* Displaced GroupNorm of one patch ([DT] corrected_async_gn, with the        */
/* reading in the header; [DF] 革命性突破 for stale reuse).                   */
/* x:      [B][C][n]  this patch's activations, this step (fresh).           */
/* stats:  [B][G][P][2] per-patch (sum, sum of squares) of the previous step. */
/* gamma, beta: [C] affine parameters, or NULL for none.                      */
/* For each (b, g), with the group's channels c in [g C/G, (g+1) C/G):        */
/*   f1 = sum_{c, i} x[b,c,i],  f2 = sum_{c, i} x[b,c,i]^2   (fresh, local)    */
/*   S1 = f1 + sum_{q != p} stats[b,g,q,0],  S2 = f2 + sum_{q != p} stats[..,1]*/
/*   N  = P * n * C/G;  mean = S1 / N;  var = S2 / N - mean^2                 */
/*   y[b,c,i] = (x[b,c,i] - mean) / sqrt(var + eps) * gamma[c] + beta[c]      */
/* fresh_out: [B][G][2] receives (f1, f2), this patch's sums for the next     */
/* step.                                                                      */
/* ------------------------------------------------------------------------ */
void oracle_displaced_group_norm(const double *x, const double *stats, const double *gamma,
                                 const double *beta, int64_t B, int64_t C, int64_t G,
                                 int64_t n, int64_t P, int64_t p, double eps, double *y,
                                 double *fresh_out)
{
    const int64_t cg = C / G;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t g = 0; g < G; ++g) {
            double f1 = 0.0, f2 = 0.0;
            for (int64_t c = g * cg; c < (g + 1) * cg; ++c)
                for (int64_t i = 0; i < n; ++i) {
                    const double v = x[(b * C + c) * n + i];
                    f1 += v;
                    f2 += v * v;
                }
            double s1 = f1, s2 = f2;
            for (int64_t q = 0; q < P; ++q)
                if (q != p) {
                    s1 += stats[((b * G + g) * P + q) * 2];
                    s2 += stats[((b * G + g) * P + q) * 2 + 1];
                }
            const double N = (double)(P * n * cg);
            const double mean = s1 / N;
            const double var = s2 / N - mean * mean;
            const double rstd = 1.0 / sqrt(var + eps);
            for (int64_t c = g * cg; c < (g + 1) * cg; ++c) {
                const double ga = gamma ? gamma[c] : 1.0, be = beta ? beta[c] : 0.0;
                for (int64_t i = 0; i < n; ++i) {
                    const int64_t k = (b * C + c) * n + i;
                    y[k] = (x[k] - mean) * rstd * ga + be;
                }
            }
            fresh_out[(b * G + g) * 2] = f1;
            fresh_out[(b * G + g) * 2 + 1] = f2;
        }
}
