/* Drives the C oracle (oracle/recurrence.c) under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every gate, key and preconditioner mode, the
 * backward, ragged and empty lengths, across the 64-token checkpoints of the
 * backward.  Host code only; exits 0 when every call returns 0 and the
 * sanitizers report nothing (they abort the process on a finding). */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_delta_rule(int B, int H, int T, int dk, int dv, const double *q, const double *k,
                      const double *v, int alpha_mode, const double *log_alpha, int beta_mode,
                      const double *beta, int gamma_mode, const double *gamma,
                      double precond_eps, const double *A0, double *AT, const double *S0,
                      double *ST, double *o, int key_mode, int precond_mode, double precond_x);
int oracle_delta_rule_bwd(int B, int H, int T, int dk, int dv, const double *q, const double *k,
                          const double *v, int alpha_mode, const double *log_alpha,
                          int beta_mode, const double *beta, int gamma_mode,
                          const double *gamma, double precond_eps, const double *A0,
                          const double *S0, int key_mode, int precond_mode, double precond_x,
                          const double *dO, const double *dST, double *dq, double *dk_out,
                          double *dv_out, double *dlog_alpha, double *dbeta, double *dgamma,
                          double *dS0, double *dA0);

static unsigned long long rng_state = 88172645463325252ULL;
static double urand(void) {  /* xorshift64, uniform in [0, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 9007199254740992.0;
}

/* exactly n doubles on the heap, so that any read past the end is reported */
static double *arr(size_t n, double lo, double hi) {
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}

static int run_case(int B, int H, int T, int dk, int dv, int am, int bm, int gm, int pre,
                    int km, int pm) {
    const size_t nq = (size_t)B * H * T * dk, nv = (size_t)B * H * T * dv;
    const size_t nbt = (size_t)B * H * T, ns = (size_t)B * H * dk * dv, na = (size_t)B * H * dk;
    double *q = arr(nq, -0.3, 0.3), *k = arr(nq, -0.3, 0.3), *v = arr(nv, -1, 1);
    double *la = am == 0 ? NULL : arr(am == 1 ? nbt : nq, -2.0, -0.01);
    double *be = arr(bm == 1 ? nbt : nq, 0.05, 1.0);
    double *ga = gm == 3 ? NULL : arr(gm == 1 ? nbt : nv, 0.05, 1.0);
    double *A0 = pre ? arr(na, 0.0, 1.0) : NULL, *AT = pre ? arr(na, 0, 0) : NULL;
    double *S0 = arr(ns, -0.1, 0.1), *ST = arr(ns, 0, 0), *o = arr(nv, 0, 0);
    int rc = oracle_delta_rule(B, H, T, dk, dv, q, k, v, am, la, bm, be, gm, ga,
                               pre ? 1e-6 : -1.0, A0, AT, S0, ST, o, km, pm, 1.5);
    double *dO = arr(nv, -1, 1), *dST = arr(ns, -1, 1);
    double *dq = arr(nq, 0, 0), *dkk = arr(nq, 0, 0), *dvv = arr(nv, 0, 0);
    double *dla = am == 0 ? NULL : arr(am == 1 ? nbt : nq, 0, 0);
    double *dbe = arr(bm == 1 ? nbt : nq, 0, 0);
    double *dga = gm == 3 ? NULL : arr(gm == 1 ? nbt : nv, 0, 0);
    double *dS0 = arr(ns, 0, 0), *dA0 = pre ? arr(na, 0, 0) : NULL;
    rc |= oracle_delta_rule_bwd(B, H, T, dk, dv, q, k, v, am, la, bm, be, gm, ga,
                                pre ? 1e-6 : -1.0, A0, S0, km, pm, 1.5, dO, dST, dq, dkk, dvv,
                                dla, dbe, dga, dS0, dA0);
    for (size_t i = 0; i < ns; ++i)
        if (!isfinite(ST[i]) || !isfinite(dS0[i])) rc |= 4;
    free(q); free(k); free(v); free(la); free(be); free(ga); free(A0); free(AT);
    free(S0); free(ST); free(o); free(dO); free(dST); free(dq); free(dkk); free(dvv);
    free(dla); free(dbe); free(dga); free(dS0); free(dA0);
    return rc;
}

int main(void) {
    int failures = 0, cases = 0;
    const int Ts[] = {0, 1, 63, 64, 65, 130};
    for (int ti = 0; ti < 6; ++ti)
        for (int am = 0; am < 3; ++am)
            for (int bm = 1; bm <= 2; ++bm)
                for (int gm = 1; gm <= 3; ++gm)
                    for (int pre = 0; pre < 2; ++pre)
                        for (int km = 0; km < 3; ++km)
                            for (int pm = 0; pm <= pre; ++pm) {
                                /* dk != dv except where a vector beta doubles as gamma */
                                const int dv = (gm == 3 && bm == 2) ? 8 : 4;
                                if (run_case(2, 1, Ts[ti], 8, dv, am, bm, gm, pre, km, pm)) {
                                    fprintf(stderr, "case T=%d a=%d b=%d g=%d pre=%d key=%d pm=%d failed\n",
                                            Ts[ti], am, bm, gm, pre, km, pm);
                                    ++failures;
                                }
                                ++cases;
                            }
    printf("oracle sanitizer driver: %d cases, %d failures\n", cases, failures);
    return failures != 0;
}
