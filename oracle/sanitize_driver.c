/*
 * sanitize_driver.c -- TEST INFRASTRUCTURE: drives every entry point of
 * gr_oracle.c over small shapes so that an AddressSanitizer / UBSan build
 * (gcc -fsanitize=address,undefined) can check the oracle's own indexing.
 * Every buffer is a separate heap block of exactly the size the function's
 * contract states, so a read or write one element past any array is caught.
 * Exit status 0 means every call returned what its contract says (0 for valid
 * arguments, -1 for rejected ones) and every output was finite.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gro_read(int64_t, int, int, int, double, int, const double *, const double *, const double *,
             const double *, const double *, double *, double *, double *, double *);
int gro_write(int64_t, int, int, int, double *, const double *, const double *);
int gro_fused(int64_t, int, int, int, double, int, double *, const double *, const double *,
              const double *, const double *, const double *, const double *, double *, double *);
int gro_add_rmsnorm(int64_t, int, double, int, double *, const double *, const double *, double *);
int gro_expand(int64_t, int, int, int, const double *, double *);
int gro_static_read(int64_t, int, int, int, const double *, const double *, double *);
int gro_round_robin_write(int64_t, int, int, int, int, double *, const double *);
int gro_write_per_channel(int64_t, int, int, int, double *, const double *, const double *);
int gro_collapse(int64_t, int, int, double, int, const double *, const double *, double *);
int gro_tanh_standin(int64_t, int, const double *, double *);
int gro_sinkhorn(int, int, const double *, double *);
int gro_hc_read(int64_t, int, int, int, int, double, int, const double *, const double *, const double *,
                const double *, const double *, const double *, double *, double *, double *);
int gro_hc_write(int64_t, int, int, int, double *, const double *, const double *);
int gro_hc_fused(int64_t, int, int, int, int, double, int, double *, const double *, const double *,
                 const double *, const double *, const double *, const double *, const double *,
                 double *, double *);
double orc_round_bf16(double);
double orc_round_e4m3(double);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;
static double urand(void)   /* splitmix64 -> uniform in [-1, 1) */
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1.0p-52 - 1.0;
}

static double *arr(int64_t count)   /* exactly `count` doubles (at least one byte) */
{
    double *p = malloc(sizeof(double) * (size_t)(count > 0 ? count : 0) + 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    for (int64_t k = 0; k < count; ++k) p[k] = urand();
    return p;
}

static int failures = 0;
static void expect(int cond, const char *what, int64_t N, int n, int d, int r, int dt)
{
    if (!cond) {
        fprintf(stderr, "FAIL %s N=%lld n=%d d=%d r=%d dtype=%d\n", what, (long long)N, n, d, r, dt);
        ++failures;
    }
}
static int finite_all(const double *p, int64_t count)
{
    for (int64_t k = 0; k < count; ++k) if (!isfinite(p[k])) return 0;
    return 1;
}

int main(void)
{
    const int ns[] = {1, 2, 3, 4, 8}, ds[] = {1, 2, 3, 8, 17}, rs[] = {0, 1, 5}, Ns[] = {0, 1, 3};
    for (int dt = 0; dt < 4; ++dt)
    for (int a = 0; a < 5; ++a) for (int b = 0; b < 5; ++b) for (int c = 0; c < 3; ++c) for (int e = 0; e < 3; ++e) {
        const int n = ns[a], d = ds[b], r = rs[c];
        const int64_t N = Ns[e], nd = (int64_t)n * d;
        double *R = arr(N * nd), *y = arr(N * d), *s_in = arr(N * n), *gamma = arr(nd);
        double *wd = r ? arr(r * nd) : NULL, *wu = r ? arr(nd * r) : NULL, *ww = arr(n * nd);
        double *u = arr(N * d), *s = arr(N * n), *rho = arr(N * n), *G = arr(N * nd);
        for (int64_t k = 0; k < N * n; ++k) s_in[k] = 1.0 + s_in[k];
        for (int with_ww = 0; with_ww < 2; ++with_ww) {
            const double *w = with_ww ? ww : NULL;
            expect(gro_read(N, n, d, r, 1e-6, dt, R, gamma, wd, wu, w, u, s, rho, G) == 0, "read", N, n, d, r, dt);
            expect(finite_all(u, N * d) && finite_all(s, N * n) && finite_all(G, N * nd), "read finite", N, n, d, r, dt);
            expect(gro_read(N, n, d, r, 1e-6, dt, R, gamma, wd, wu, w, u, NULL, NULL, NULL) == 0, "read (no s)", N, n, d, r, dt);
            double *Rc = arr(N * nd);
            memcpy(Rc, R, sizeof(double) * (size_t)(N * nd));
            expect(gro_fused(N, n, d, r, 1e-6, dt, Rc, y, s_in, gamma, wd, wu, w, u, s) == 0, "fused", N, n, d, r, dt);
            expect(finite_all(Rc, N * nd) && finite_all(u, N * d), "fused finite", N, n, d, r, dt);
            free(Rc);
        }
        expect(gro_write(N, n, d, dt, R, y, s_in) == 0, "write", N, n, d, r, dt);
        double *e0 = arr(N * d), *h = arr(n), *sc = arr(nd), *w1 = arr(d), *o = arr(N * d);
        expect(gro_expand(N, n, d, dt, e0, R) == 0, "expand", N, n, d, r, dt);
        expect(gro_static_read(N, n, d, dt, R, h, o) == 0, "static_read", N, n, d, r, dt);
        expect(gro_round_robin_write(N, n, d, 7, dt, R, y) == 0, "round_robin_write", N, n, d, r, dt);
        expect(gro_write_per_channel(N, n, d, dt, R, y, sc) == 0, "write_per_channel", N, n, d, r, dt);
        expect(gro_collapse(N, n, d, 1e-6, dt, R, w1, o) == 0, "collapse", N, n, d, r, dt);
        double *x = arr(N * d);
        expect(gro_add_rmsnorm(N, d, 1e-6, dt, x, y, w1, o) == (dt == 3 ? -1 : 0), "add_rmsnorm", N, n, d, r, dt);
        expect(gro_tanh_standin(N * d, dt, u, o) == 0, "tanh_standin", N, n, d, r, dt);
        /* HC / mHC: coefficient records of n + n*n, projections of n + 2 rows */
        {
            const int64_t nc = n + (int64_t)n * n;
            double *P = arr((n + 2) * (int64_t)d), *hs = arr(2 * n + (int64_t)n * n), *lam = arr(3);
            double *cin = arr(N * nc), *cout = arr(N * nc), *hm = arr(N * n), *uu = arr(N * d);
            double *L = arr((int64_t)n * n), *M = arr((int64_t)n * n);
            expect(gro_sinkhorn(n, 20, L, M) == 0 && finite_all(M, (int64_t)n * n), "sinkhorn", N, n, d, r, dt);
            for (int mode = 0; mode < 2; ++mode) {
                expect(gro_hc_read(N, n, d, mode, 20, 1e-6, dt, R, gamma, w1, P, hs, lam, uu, cout, hm) == 0,
                       "hc_read", N, n, d, r, dt);
                expect(finite_all(uu, N * d) && finite_all(cout, N * nc) && finite_all(hm, N * n),
                       "hc_read finite", N, n, d, r, dt);
                expect(gro_hc_fused(N, n, d, mode, 20, 1e-6, dt, R, y, cin, gamma, w1, P, hs, lam, uu, cout) == 0,
                       "hc_fused", N, n, d, r, dt);
            }
            expect(gro_hc_write(N, n, d, dt, R, y, cin) == 0, "hc_write", N, n, d, r, dt);
            expect(gro_hc_read(N, n, d, 2, 20, 1e-6, dt, R, gamma, w1, P, hs, lam, uu, cout, NULL) == -1,
                   "hc_read bad mode", N, n, d, r, dt);
            free(P); free(hs); free(lam); free(cin); free(cout); free(hm); free(uu); free(L); free(M);
        }
        free(R); free(y); free(s_in); free(gamma); free(wd); free(wu); free(ww); free(u); free(s);
        free(rho); free(G); free(e0); free(h); free(sc); free(w1); free(o); free(x);
    }
    /* rejected arguments return -1 without touching memory */
    expect(gro_read(1, 0, 4, 0, 1e-6, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == -1, "read n=0", 1, 0, 4, 0, 1);
    expect(gro_read(1, 2, 4, 3, 1e-6, 1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == -1, "read r>0 without W", 1, 2, 4, 3, 1);
    expect(gro_write(-1, 2, 4, 1, NULL, NULL, NULL) == -1, "write N<0", -1, 2, 4, 0, 1);
    expect(gro_round_robin_write(1, 2, 4, -1, 1, NULL, NULL) == -1, "round robin layer<0", 1, 2, 4, 0, 1);
    /* rounding helpers over extremes */
    const double xs[] = {0.0, -0.0, 1e-45, -1e-300, 3.4e38, -3.5e38, 1e308, 448.0, 449.0, -1e9, 0x1.0p-133};
    for (size_t k = 0; k < sizeof xs / sizeof xs[0]; ++k) {
        (void)orc_round_bf16(xs[k]);
        expect(fabs(orc_round_e4m3(xs[k])) <= 448.0, "e4m3 saturates", 0, 0, 0, 0, 3);
    }
    if (failures) { fprintf(stderr, "%d failure(s)\n", failures); return 1; }
    printf("sanitized oracle: all calls ok\n");
    return 0;
}
