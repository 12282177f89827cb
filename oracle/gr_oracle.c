/*
 * gr_oracle.c -- TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, slow, single-threaded fp64 evaluation of the Gated Residual (GR)
 * read and write, of the fused write+read, and of the n = 1 fused residual
 * add + RMSNorm.  It exists to check the HIP path; only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Sources (cited by page title and section / equation):
 *   [QFN]  "Paper reading: Qwen3.8 Flash Next" (wkq9411.github.io), part 2
 *          "Residual", section 4 "Gated Residual (GR)": eq:rms, eq:gate,
 *          eq:use_gate, eq:s, eq:write.
 *   [NOTES] "Qwen3.8-Flash-Next architecture notes, 06 Residual"
 *          (cbphcr.github.io), section 2 (GR read) and section 3 (GR write):
 *          the same equations restated with n_r = 4.
 *   [RES]  "Residual" (rainlin-net.pages.dev, LLM inference), section 2.2
 *          (Pre-Norm) and section 3.3 (fused residual add + RMSNorm).
 *   [QFN sec. 1] the AltUp-style static read (eq:input) and round-robin write
 *          (eq:output); [QFN sec. 6] eq:rcv (branches start at the embedding).
 *
 * Conventions adopted where the pages leave a point open:
 *   - RMSNorm(x; g)_c = g_c * x_c / sqrt(mean(x^2) + eps), eps inside the root;
 *     g is the effective gain (a zero-centred model passes 1 + g).
 *   - vec() stacks branches: vec index of (branch i, channel c) is i*d + c;
 *     W_down is [r][n*d], W_up is [n*d][r], W_write is [n][n*d], row-major.
 *   - r == 0 means a unit gate (G == 1); W_write == NULL means s == 1.
 *   - All arithmetic is fp64.  Results are rounded to the storage dtype only
 *     where the path stores them: the state, u, and (for the chain) F's y;
 *     s is rounded to fp32.  Storage dtype 2 ("f64") skips that rounding, for
 *     exact closed-form checks.
 *   - Storage dtype 3 ("fp8"): the branch state is OCP e4m3 (e4m3fn: 3
 *     mantissa bits, no infinities, largest finite 448), everything else --
 *     u, y, gains, weights -- is bf16.  [QFN sec. 7] names an FP8 state
 *     without a format or a scale: unscaled e4m3 is the reading, and a value
 *     beyond +-448 saturates to +-448 (e4m3fn has no infinity; a NaN would
 *     poison the residual stream).
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2, ORC_FP8 = 3 };

/* Largest finite bfloat16: (2 - 2^-7) * 2^127. */
#define ORC_BF16_MAX 3.3895313892515355e38

/* Round x to the nearest bfloat16 (8 significant bits, fp32 exponent range),
 * ties to even.  Below 2^-126 the spacing is the fixed subnormal step 2^-133. */
double orc_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                  /* |x| in [2^(e-1), 2^e) */
    int q = e - 8;                 /* spacing of 8-bit significands there */
    if (q < -133) q = -133;
    double y = ldexp(nearbyint(ldexp(x, -q)), q);   /* nearbyint: ties-to-even */
    if (fabs(y) > ORC_BF16_MAX) return copysign(INFINITY, x);
    return y;
}

/* Round x to the nearest fp32 (C conversion under the default rounding mode). */
double orc_round_f32(double x) { return (double)(float)x; }

/* Round x to the nearest OCP e4m3 value (4 significant bits, exponent bias 7,
 * subnormal step 2^-9 below 2^-6), ties to even; magnitudes beyond the largest
 * finite value 448 saturate to +-448. */
double orc_round_e4m3(double x)
{
    if (x == 0.0 || isnan(x)) return x;
    if (fabs(x) >= 448.0) return copysign(448.0, x);
    int e;
    frexp(x, &e);                  /* |x| in [2^(e-1), 2^e) */
    int q = e - 4;                 /* spacing of 4-bit significands there */
    if (q < -9) q = -9;
    double y = ldexp(nearbyint(ldexp(x, -q)), q);   /* nearbyint: ties-to-even */
    if (fabs(y) > 448.0) return copysign(448.0, x);
    return y;
}

/* Stores of the branch state. */
static double store_state(double x, int dtype)
{
    if (dtype == ORC_BF16) return orc_round_bf16(x);
    if (dtype == ORC_F32) return orc_round_f32(x);
    if (dtype == ORC_FP8) return orc_round_e4m3(x);
    return x;
}

/* Stores of everything else (u, the chain's y, add+RMSNorm's outputs). */
static double store_round(double x, int dtype)
{
    if (dtype == ORC_BF16 || dtype == ORC_FP8) return orc_round_bf16(x);
    if (dtype == ORC_F32) return orc_round_f32(x);
    return x;
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }
static double silu(double x) { return x * sigmoid(x); }

/*
 * GR read for N tokens  [QFN eq:rms, eq:gate, eq:use_gate, eq:s; NOTES sec. 2-3].
 *
 *   R      [N][n][d]   state (exact stored values)
 *   gamma  [n][d]      per-branch RMSNorm gains
 *   wd     [r][n*d]    down projection (NULL iff r == 0)
 *   wu     [n*d][r]    up projection   (NULL iff r == 0)
 *   ww     [n][n*d]    write projection, or NULL for unit write strengths
 *   u      [N][d]      out: sublayer input x (rounded to the storage dtype)
 *   s      [N][n]      out: write strengths (rounded to fp32); may be NULL
 *   rho    [N][n]      out (optional): 1/rms of each branch
 *   gate   [N][n][d]   out (optional): G
 * Returns 0, or -1 on bad sizes / allocation failure.
 */
int gro_read(int64_t N, int n, int d, int r, double eps, int dtype,
             const double *R, const double *gamma, const double *wd,
             const double *wu, const double *ww, double *u, double *s,
             double *rho, double *gate)
{
    if (N < 0 || n < 1 || d < 1 || r < 0) return -1;
    if (r > 0 && (!wd || !wu)) return -1;
    const int64_t nd = (int64_t)n * d;
    double *vhat = malloc(sizeof(double) * nd);      /* vec(R-hat) */
    double *g = malloc(sizeof(double) * nd);         /* G, vec order */
    double *a = malloc(sizeof(double) * (r > 0 ? r : 1));
    double *rh = malloc(sizeof(double) * n);
    if (!vhat || !g || !a || !rh) { free(vhat); free(g); free(a); free(rh); return -1; }

    for (int64_t t = 0; t < N; ++t) {
        const double *Rt = R + t * nd;
        /* eq:rms -- each branch normalised on its own, with its own gain. */
        for (int i = 0; i < n; ++i) {
            double ss = 0.0;
            for (int c = 0; c < d; ++c) ss += Rt[i * d + c] * Rt[i * d + c];
            rh[i] = 1.0 / sqrt(ss / d + eps);
            for (int c = 0; c < d; ++c)
                vhat[i * d + c] = gamma[i * d + c] * Rt[i * d + c] * rh[i];
        }
        /* eq:gate -- G = unvec sigmoid(W_up SiLU((1/n) W_down vec(R-hat))). */
        if (r > 0) {
            for (int k = 0; k < r; ++k) {
                double acc = 0.0;
                for (int64_t j = 0; j < nd; ++j) acc += wd[k * nd + j] * vhat[j];
                a[k] = silu(acc / n);
            }
            for (int64_t j = 0; j < nd; ++j) {
                double acc = 0.0;
                for (int k = 0; k < r; ++k) acc += wu[j * r + k] * a[k];
                g[j] = sigmoid(acc);
            }
        } else {
            for (int64_t j = 0; j < nd; ++j) g[j] = 1.0;
        }
        /* eq:use_gate -- x = (1/n) sum_i G_i (.) R-hat_i. */
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i) acc += g[i * d + c] * vhat[i * d + c];
            u[t * d + c] = store_round(acc / n, dtype);
        }
        /* eq:s -- s = 2 sigmoid((1/n) W_write vec(R-hat)). */
        if (s) {
            for (int i = 0; i < n; ++i) {
                double val = 1.0;
                if (ww) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < nd; ++j) acc += ww[i * nd + j] * vhat[j];
                    val = 2.0 * sigmoid(acc / n);
                }
                s[t * n + i] = dtype == ORC_F64 ? val : orc_round_f32(val);
            }
        }
        if (rho) for (int i = 0; i < n; ++i) rho[t * n + i] = rh[i];
        if (gate) memcpy(gate + t * nd, g, sizeof(double) * nd);
    }
    free(vhat); free(g); free(a); free(rh);
    return 0;
}

/*
 * GR write for N tokens  [QFN eq:write; NOTES sec. 3]:
 *   R'_i = R_i + s_i * y, the same y into every branch, stored in place.
 *   R [N][n][d] in/out, y [N][d], s [N][n].
 * The pages fix no precision for forming R + s y before it is stored; the
 * workloads state their arithmetic as a bf16 (or e4m3) state with fp32
 * accumulation, and adding s y into the state is that accumulation.  So the
 * sum (exact in fp64 here whenever it can matter) is rounded to fp32 -- what
 * one fp32 fused multiply-add delivers -- and that fp32 value is stored, i.e.
 * rounded again to the storage dtype.  Where this differs from one rounding
 * of the exact sum (the fp32 value sits exactly on a rounding midpoint of the
 * storage dtype) the two differ by one unit in the last place.
 */
int gro_write(int64_t N, int n, int d, int dtype, double *R, const double *y,
              const double *s)
{
    if (N < 0 || n < 1 || d < 1) return -1;
    for (int64_t t = 0; t < N; ++t)
        for (int i = 0; i < n; ++i)
            for (int c = 0; c < d; ++c) {
                double *p = R + (t * n + i) * (int64_t)d + c;
                const double sum = *p + s[t * n + i] * y[t * d + c];
                *p = store_state(dtype == ORC_F64 ? sum : orc_round_f32(sum), dtype);
            }
    return 0;
}

/*
 * Fused write of one sublayer followed by the read of the next
 * [QFN sec. 2.7 (one traversal per direction), eq:write then eq:rms..eq:s]:
 * the write is completed and stored first; the read then sees the stored R'.
 */
int gro_fused(int64_t N, int n, int d, int r, double eps, int dtype, double *R,
              const double *y, const double *s_in, const double *gamma,
              const double *wd, const double *wu, const double *ww, double *u,
              double *s_out)
{
    int rc = gro_write(N, n, d, dtype, R, y, s_in);
    if (rc) return rc;
    return gro_read(N, n, d, r, eps, dtype, R, gamma, wd, wu, ww, u, s_out, NULL, NULL);
}

/*
 * n = 1 fused residual add + RMSNorm  [RES sec. 3.3]:
 *   h = x + y (stored in place of x), out = w (.) h / sqrt(mean(h^2) + eps),
 *   the norm taken over the stored h.  x, y, out [N][d], w [d].
 */
int gro_add_rmsnorm(int64_t N, int d, double eps, int dtype, double *x,
                    const double *y, const double *w, double *out)
{
    if (N < 0 || d < 1 || dtype == ORC_FP8) return -1;
    for (int64_t t = 0; t < N; ++t) {
        double *h = x + t * d;
        double ss = 0.0;
        for (int c = 0; c < d; ++c) {
            h[c] = store_round(h[c] + y[t * d + c], dtype);
            ss += h[c] * h[c];
        }
        double inv = 1.0 / sqrt(ss / d + eps);
        for (int c = 0; c < d; ++c) out[t * d + c] = store_round(w[c] * h[c] * inv, dtype);
    }
    return 0;
}

/*
 * Variants on the same widened state (the f4 row of the hot-path table).
 *
 * Expand  [QFN sec. 6, eq:rcv: the initial value of every branch is the token
 * embedding]: R[t][i][c] = e[t][c] for every branch i, stored in the state
 * dtype.  e [N][d], R [N][n][d].
 */
int gro_expand(int64_t N, int n, int d, int dtype, const double *e, double *R)
{
    if (N < 0 || n < 1 || d < 1) return -1;
    for (int64_t t = 0; t < N; ++t)
        for (int i = 0; i < n; ++i)
            for (int c = 0; c < d; ++c)
                R[(t * n + i) * (int64_t)d + c] = store_state(e[t * d + c], dtype);
    return 0;
}

/*
 * Static read  [QFN sec. 1, eq:input: the AltUp-style block input is a
 * weighted sum of the branches with n learned scalars]:
 *   u[t][c] = sum_i h[i] R[t][i][c], stored in the dtype of u.
 */
int gro_static_read(int64_t N, int n, int d, int dtype, const double *R, const double *h,
                    double *u)
{
    if (N < 0 || n < 1 || d < 1) return -1;
    for (int64_t t = 0; t < N; ++t)
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i) acc += h[i] * R[(t * n + i) * (int64_t)d + c];
            u[t * d + c] = store_round(acc, dtype);
        }
    return 0;
}

/*
 * Round-robin write  [QFN sec. 1, eq:output: the block output is added to one
 * branch, chosen by depth in turn, the others unchanged]:
 *   R[t][layer mod n][c] += y[t][c].
 * The sum is rounded as eq:write's (through fp32, then the state dtype).
 */
int gro_round_robin_write(int64_t N, int n, int d, int layer, int dtype, double *R,
                          const double *y)
{
    if (N < 0 || n < 1 || d < 1 || layer < 0) return -1;
    const int i = layer % n;
    for (int64_t t = 0; t < N; ++t)
        for (int c = 0; c < d; ++c) {
            double *p = R + (t * n + i) * (int64_t)d + c;
            const double sum = *p + y[t * d + c];
            *p = store_state(dtype == ORC_F64 ? sum : orc_round_f32(sum), dtype);
        }
    return 0;
}

/*
 * Per-channel write  [NOTES sec. 3: a per-channel write was tried in place of
 * the per-branch scalar]: the pages give no formula for predicting per-channel
 * strengths, so they are a learned [n][d] parameter here:
 *   R'[t][i][c] = R[t][i][c] + s[i][c] y[t][c],
 * rounded as eq:write's.
 */
int gro_write_per_channel(int64_t N, int n, int d, int dtype, double *R, const double *y,
                          const double *s)
{
    if (N < 0 || n < 1 || d < 1) return -1;
    for (int64_t t = 0; t < N; ++t)
        for (int i = 0; i < n; ++i)
            for (int c = 0; c < d; ++c) {
                double *p = R + (t * n + i) * (int64_t)d + c;
                const double sum = *p + s[i * (int64_t)d + c] * y[t * d + c];
                *p = store_state(dtype == ORC_F64 ? sum : orc_round_f32(sum), dtype);
            }
    return 0;
}

/*
 * Collapse  (the pages describe no read-out of the widened stream after the
 * last GR block; the nearest statement, for a four-stream residual, sums the
 * streams and then applies RMSNorm): h = sum_i R_i (not stored), then
 *   out[t][c] = w[c] h[c] / sqrt(mean_c h^2 + eps), stored in the dtype of u.
 */
int gro_collapse(int64_t N, int n, int d, double eps, int dtype, const double *R,
                 const double *w, double *out)
{
    if (N < 0 || n < 1 || d < 1) return -1;
    double *h = malloc(sizeof(double) * d);
    if (!h) return -1;
    for (int64_t t = 0; t < N; ++t) {
        double ss = 0.0;
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i) acc += R[(t * n + i) * (int64_t)d + c];
            h[c] = acc;
            ss += acc * acc;
        }
        const double inv = 1.0 / sqrt(ss / d + eps);
        for (int c = 0; c < d; ++c) out[t * d + c] = store_round(w[c] * h[c] * inv, dtype);
    }
    free(h);
    return 0;
}

/* Elementwise sublayer stand-in of the chained workload: y = 0.1 tanh(u). */
int gro_tanh_standin(int64_t count, int dtype, const double *u, double *y)
{
    if (count < 0) return -1;
    for (int64_t k = 0; k < count; ++k) y[k] = store_round(0.1 * tanh(u[k]), dtype);
    return 0;
}

/* ------------------------------------------------------------------------
 * Hyper-Connections (HC) and manifold-constrained HC (mHC)
 *
 * [QFN sec. 2] "Hyper-Connections": a block reads x = H_mix^T R, runs
 * y = F(Norm(x)) (eq:block), and writes R' = H_res R + H_combine y^T, with
 * H_mix, H_combine in R^n and H_res in R^{n x n}.  Each operator is a static
 * term plus a data-dependent term predicted from the normalised branches
 * Rbar = Norm(R): H = H^s + lambda * phi(Rbar W) (eq:mix, eq:combine and the
 * line after them); HC takes phi = tanh.
 * [DB sec. 2.5] "DepthBench" (cc.laoqi.cc), "Block AttnRes and mHC": mHC reads
 * with sigmoid weights, writes with twice-sigmoid weights, and maps the
 * propagation matrix through 20 Sinkhorn-Knopp iterations to an approximately
 * doubly stochastic one.
 *
 * Readings where the pages leave a point open:
 *   - Norm is the per-branch RMSNorm of eq:rms: Rbar_i = g_i * R_i * rho_i,
 *     rho_i = 1/sqrt(mean_c R_ic^2 + eps), with a gain g_i per branch.
 *   - Rbar W_m, Rbar W_c are n-vectors and Rbar W_r an n x n matrix, so
 *     W_m, W_c are d-vectors and W_r is d x n, shared by the branches:
 *     (Rbar W_r)_ij = sum_c Rbar_ic W_r[c][j].  They are passed as the rows
 *     of P [n+2][d]: P[0] = W_m, P[1] = W_c, P[2+j] = column j of W_r.
 *   - lambda_m, lambda_c, lambda_r are scalars.
 *   - HC:  H_mix = Hs_mix + lm tanh(Rbar W_m), H_comb = Hs_comb + lc tanh(Rbar W_c),
 *          H_res = Hs_res + lr tanh(Rbar W_r).
 *   - mHC: H_mix = sigmoid(Hs_mix + lm Rbar W_m), H_comb = 2 sigmoid(Hs_comb + lc Rbar W_c),
 *          H_res = SK(exp(Hs_res + lr Rbar W_r)): exp makes the matrix positive,
 *          as Sinkhorn-Knopp requires; one iteration divides every row by its
 *          sum, then every column by its sum.
 *   - The block's Norm is an RMSNorm with gain w: u = w x / sqrt(mean x^2 + eps),
 *     stored in the state dtype; x is formed from the raw R (eq:block).
 *   - The read predicts all three operators from the same pre-write state; it
 *     hands H_combine and H_res (the coefficient record [H_comb | H_res row-major],
 *     n + n*n values, fp32) to the write of the same block, as the GR read
 *     hands s to its write.
 *   - The write is evaluated exactly (fp64) and rounded once to the state dtype.
 * ------------------------------------------------------------------------ */

enum { ORC_HC_TANH = 0, ORC_HC_MHC = 1 };

/* Sinkhorn-Knopp [DB sec. 2.5]: M = exp(L) (n x n, row-major), then `iters`
 * times: scale each row to sum 1, then each column to sum 1. */
int gro_sinkhorn(int n, int iters, const double *L, double *M)
{
    if (n < 1 || iters < 0) return -1;
    for (int k = 0; k < n * n; ++k) M[k] = exp(L[k]);
    for (int it = 0; it < iters; ++it) {
        for (int i = 0; i < n; ++i) {
            double s = 0.0;
            for (int j = 0; j < n; ++j) s += M[i * n + j];
            for (int j = 0; j < n; ++j) M[i * n + j] /= s;
        }
        for (int j = 0; j < n; ++j) {
            double s = 0.0;
            for (int i = 0; i < n; ++i) s += M[i * n + j];
            for (int i = 0; i < n; ++i) M[i * n + j] /= s;
        }
    }
    return 0;
}

/*
 * HC / mHC read of one block.
 *   R [N][n][d]; g [n][d]; w [d]; P [n+2][d]; hs [2n + n*n] = Hs_mix | Hs_comb | Hs_res;
 *   lam[3] = lambda_m, lambda_c, lambda_r.
 * Outputs u [N][d] (state dtype), coeff [N][n + n*n] (fp32), and, if given,
 * hmix [N][n] (fp64, for tests).
 */
int gro_hc_read(int64_t N, int n, int d, int mode, int iters, double eps, int dtype,
                const double *R, const double *g, const double *w, const double *P,
                const double *hs, const double *lam, double *u, double *coeff, double *hmix)
{
    if (N < 0 || n < 1 || d < 1 || (mode != ORC_HC_TANH && mode != ORC_HC_MHC)) return -1;
    const int nc = n + n * n;
    double *rbar = malloc(sizeof(double) * n * d);
    double *proj = malloc(sizeof(double) * n * (n + 2));   /* proj[i][k] = Rbar_i . P[k] */
    double *hm = malloc(sizeof(double) * n);
    double *L = malloc(sizeof(double) * n * n);
    double *Hres = malloc(sizeof(double) * n * n);
    double *x = malloc(sizeof(double) * d);
    if (!rbar || !proj || !hm || !L || !Hres || !x) {
        free(rbar); free(proj); free(hm); free(L); free(Hres); free(x);
        return -1;
    }
    for (int64_t t = 0; t < N; ++t) {
        const double *Rt = R + t * n * (int64_t)d;
        /* Rbar = per-branch RMSNorm (eq:rms) */
        for (int i = 0; i < n; ++i) {
            double ss = 0.0;
            for (int c = 0; c < d; ++c) ss += Rt[i * d + c] * Rt[i * d + c];
            const double rho = 1.0 / sqrt(ss / d + eps);
            for (int c = 0; c < d; ++c) rbar[i * d + c] = g[i * d + c] * Rt[i * d + c] * rho;
        }
        for (int i = 0; i < n; ++i)
            for (int k = 0; k < n + 2; ++k) {
                double acc = 0.0;
                for (int c = 0; c < d; ++c) acc += rbar[i * d + c] * P[k * (int64_t)d + c];
                proj[i * (n + 2) + k] = acc;
            }
        double *ct = coeff + t * nc;
        for (int i = 0; i < n; ++i) {
            const double am = proj[i * (n + 2) + 0], ac = proj[i * (n + 2) + 1];
            if (mode == ORC_HC_TANH) {
                hm[i] = hs[i] + lam[0] * tanh(am);
                ct[i] = hs[n + i] + lam[1] * tanh(ac);
            } else {
                hm[i] = sigmoid(hs[i] + lam[0] * am);
                ct[i] = 2.0 * sigmoid(hs[n + i] + lam[1] * ac);
            }
            for (int j = 0; j < n; ++j) {
                const double ar = proj[i * (n + 2) + 2 + j];
                if (mode == ORC_HC_TANH) Hres[i * n + j] = hs[2 * n + i * n + j] + lam[2] * tanh(ar);
                else L[i * n + j] = hs[2 * n + i * n + j] + lam[2] * ar;
            }
        }
        if (mode == ORC_HC_MHC) gro_sinkhorn(n, iters, L, Hres);
        for (int i = 0; i < n; ++i) ct[i] = orc_round_f32(ct[i]);
        for (int k = 0; k < n * n; ++k) ct[n + k] = orc_round_f32(Hres[k]);
        if (hmix) for (int i = 0; i < n; ++i) hmix[t * n + i] = hm[i];
        /* x = H_mix^T R, then the block's RMSNorm (eq:block) */
        double ss = 0.0;
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int i = 0; i < n; ++i) acc += hm[i] * Rt[i * d + c];
            x[c] = acc;
            ss += acc * acc;
        }
        const double inv = 1.0 / sqrt(ss / d + eps);
        for (int c = 0; c < d; ++c) u[t * d + c] = store_round(w[c] * x[c] * inv, dtype);
    }
    free(rbar); free(proj); free(hm); free(L); free(Hres); free(x);
    return 0;
}

/* HC / mHC write [QFN sec. 2]: R'_i = sum_j H_res[i][j] R_j + H_comb[i] y, with
 * coeff [N][n + n*n] = H_comb | H_res row-major; exact, then one rounding. */
int gro_hc_write(int64_t N, int n, int d, int dtype, double *R, const double *y,
                 const double *coeff)
{
    if (N < 0 || n < 1 || d < 1) return -1;
    const int nc = n + n * n;
    double *old = malloc(sizeof(double) * n);
    if (!old) return -1;
    for (int64_t t = 0; t < N; ++t) {
        double *Rt = R + t * n * (int64_t)d;
        const double *ct = coeff + t * nc;
        for (int c = 0; c < d; ++c) {
            for (int j = 0; j < n; ++j) old[j] = Rt[j * d + c];
            for (int i = 0; i < n; ++i) {
                double acc = ct[i] * y[t * d + c];
                for (int j = 0; j < n; ++j) acc += ct[n + i * n + j] * old[j];
                Rt[i * d + c] = store_state(acc, dtype);
            }
        }
    }
    free(old);
    return 0;
}

/* Write of block l (coefficients coeff_in), then the read of block l+1 on the
 * stored state. */
int gro_hc_fused(int64_t N, int n, int d, int mode, int iters, double eps, int dtype,
                 double *R, const double *y, const double *coeff_in, const double *g,
                 const double *w, const double *P, const double *hs, const double *lam,
                 double *u, double *coeff_out)
{
    int rc = gro_hc_write(N, n, d, dtype, R, y, coeff_in);
    if (rc) return rc;
    return gro_hc_read(N, n, d, mode, iters, eps, dtype, R, g, w, P, hs, lam, u, coeff_out, NULL);
}
